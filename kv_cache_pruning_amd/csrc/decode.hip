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
// Launch 1, decode_token_kernel (B + 1 workgroups): everything that depends
// on the token alone, once per sequence -- the gate projection x [W_dec |
// W_dn], the log-gates of every KV head, the output gate sigmoid(u W_up +
// b_up) of every query head, the rotated queries, the stored key (normalised,
// rotated, rounded like the cache) and the token's logit against its own key
// -- written to the workspace.  The last workgroup numbers the tiles of the
// step from the segment lengths (a tile is TWG consecutive entries of one
// segment), writes one record per tile, and clears the per-segment counters
// and the look-back words of the second launch.
//
// Launch 2, decode_tile_kernel (one workgroup per possible tile, four waves):
// a workgroup past the step's tile count exits at once; the others read their
// tile record, issue every cache load of the tile together with the token's
// rotated queries and key, and read each entry once: the key row feeds the G
// query dot products and the key-similarity dot product (reduced over the
// d/8 lanes that hold the row, with DPP), the pair term updates the log-bias,
// entries below log p drop out, and an online-softmax partial (max, sum,
// weighted V) is formed per wave and merged across the waves in LDS.  The
// workgroups of a segment's tiles draw the tile numbers from a per-segment
// ticket, so a tile's predecessors in its segment are held by workgroups that
// started earlier: every wait below is on one of them.
//  * A one-tile segment combines at once; otherwise each tile publishes its
//    partial and the last to arrive (an atomic counter) merges them.  The
//    combine adds the token's own term and multiplies by the output gate.
//  * With COMPACT the survivors move down in place: a tile publishes its live
//    count once every row of the tile is in registers and looks back over the
//    earlier tiles of its segment for its destination (decoupled look-back);
//    the look-back cannot finish before every earlier tile has published,
//    which orders the stores after the loads they overwrite.  Rows already in
//    place are not rewritten; every survivor's new log-bias is stored.  The
//    segment's last tile learns the new length, appends the new entry after
//    the survivors and writes the length.
//  * Without COMPACT the log-biases are updated in place and the segment's
//    first tile appends the new entry at the old length.
// No launch reads a length another workgroup of the same launch writes: the
// tile records carry the lengths at the start of the step.
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

constexpr int kTokThreads = 256;
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
constexpr int decode_nb(int d, int g) { return g >= 8 ? 2 : 4; }

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
};

// ---------------------------------------------------------------------------
// launch 1: the token's own quantities, once per sequence; the tile records
// ---------------------------------------------------------------------------
// z[c] = x . M[:, c] for the ncols columns of a row-major [D, ncols] matrix,
// into s_z.  Threads take 16-byte column chunks (or single columns) and split
// the rows; partial sums meet in LDS.
template <bool BF16>
__device__ void token_gemv(const LayerArgs& a, const void* Mv, int ncols, const char* xrow, float* s_z,
                           float (*s_red)[8]) {
  constexpr int CW = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int NT = kTokThreads;
  constexpr int KR = 16;  // rows per thread per pass, all loads in flight together
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int Dm = a.D_model;
  const char* const mbase = reinterpret_cast<const char*>(Mv);
  const bool vec = ncols % CW == 0;
  const int nch = vec ? ncols / CW : ncols;  // column groups (16-byte chunks or single columns)
  int npow = 1;
  while (npow < nch) npow <<= 1;
  const int R = NT / npow;  // row subsets (>= 1: ncols <= 3 * 64 + 64 columns)
  const int kc = tid & (npow - 1), rsub = tid / npow;
  const bool own = kc < nch;
  const int mc0 = own ? (vec ? kc * CW : kc) : 0;
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
  int reff;
  if (npow <= 64) {  // a wave holds every column group: reduce its row subsets in registers
    for (int o = npow; o < 64; o <<= 1) {
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] += __shfl_xor(acc[t], o, 64);
    }
    if (lane < npow) {
#pragma unroll
      for (int t = 0; t < 8; ++t) s_red[wv * npow + lane][t] = acc[t];
    }
    reff = NT / 64;
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) s_red[tid][t] = acc[t];
    reff = R;
  }
  __syncthreads();
  for (int c = tid; c < ncols; c += NT) {
    const int grp = vec ? c / CW : c;
    const int t = vec ? c % CW : 0;
    float z = 0.0f;
    for (int rr = 0; rr < reff; ++rr) z += s_red[rr * npow + grp][t];
    s_z[c] = z;
  }
  __syncthreads();
}

template <int D, bool BF16>
__global__ __launch_bounds__(kTokThreads) void decode_token_kernel(DecodeKArgs karg) {
  const DecodeKArgs& K = *(const DecodeKArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const LayerArgs& a = K.a;
  const DecodeWs& w = K.w;
  constexpr int NT = kTokThreads;
  constexpr int HALF = D / 2;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int Hkv = a.H_kv, Hq = a.H_q, G = Hq / Hkv;
  const int S = a.B * Hkv;
  const int b = blockIdx.x;

  __shared__ float s_red[NT][8];
  __shared__ float s_z[3 * kMaxHkv + kMaxRank];
  __shared__ float s_cs[HALF], s_sn[HALF];
  __shared__ int s_scan[NT / 64 + 1];

  if (b == a.B) {
    // ---- the tile records of this step, from the lengths at its start
    const int twg = K.twg;
    const int per = (S + NT - 1) / NT;
    const int sb = min(S, tid * per), se = min(S, sb + per);
    int mine = 0;
    for (int s = sb; s < se; ++s) mine += tiles_of(a.seg_len[s], twg);
    int total;
    int run = block_exclusive_scan<NT>(mine, s_scan, &total);
    for (int s = sb; s < se; ++s) {
      const int len = a.seg_len[s];
      const int nt = tiles_of(len, twg);
      const int64_t off = a.seg_off[s];
      for (int t = 0; t < nt && run + t < w.max_tiles; ++t) {  // lengths beyond capacity break the bound
        w.map[2 * (run + t) + 0] = make_int4(s, t, len, nt);
        w.map[2 * (run + t) + 1] = make_int4(run, (int)(uint32_t)(off & 0xffffffff), (int)(off >> 32), 0);
      }
      w.cnt[s] = 0;
      w.segtk[s] = 0;
      run += nt;
    }
    if (total > w.max_tiles) {  // a segment length above its capacity: no tile runs
      if (tid == 0) atomicOr(a.status, 4);
      total = 0;
    }
    for (int t = tid; t < total; t += NT) K.ctl.dec_state[t] = 0ull;
    if (tid == 0) *w.ntiles = total;
    return;
  }

  // ---- sequence b: position, RoPE table (fp64 angles)
  const int pos = a.next_pos[b];
  if (tid < HALF) {
    double sn, cs;
    sincos((double)pos * a.inv_freq[tid], &sn, &cs);
    s_cs[tid] = (float)cs;
    s_sn[tid] = (float)sn;
  }
  // ---- gate projection x [W_dec | W_dn]
  const char* const xrow = reinterpret_cast<const char*>(a.x) + (int64_t)b * a.D_model * (BF16 ? 2 : 4);
  token_gemv<BF16>(a, a.W_dec, 3 * Hkv, xrow, s_z, s_red);
  token_gemv<BF16>(a, a.W_dn, a.r, xrow, s_z + 3 * Hkv, s_red);
  if (tid == 0) a.next_pos[b] = pos + 1;

  // ---- per KV head: the query/similarity part of the pair term (log2 units,
  // divided by the number of enabled terms) and the new key's gate
  const PairCoef pc = pair_coef(a.terms);
  for (int h = tid; h < Hkv; h += NT) {
    const float lq = log_sigmoid(s_z[h] + a.b_dec[h]);
    const float lkn = log_sigmoid(s_z[Hkv + h] + a.b_dec[Hkv + h]);
    const float lb = log_sigmoid(s_z[2 * Hkv + h] + a.b_dec[2 * Hkv + h]);
    const float row2 = (((a.terms & 1) ? lq : 0.0f) + ((a.terms & 4) ? lb : 0.0f)) * pc.inv_n2;
    w.tokf[(b * Hkv + h) * 2 + 0] = row2;
    w.tokf[(b * Hkv + h) * 2 + 1] = lkn;
  }
  // ---- output gate of every query head: sigmoid(u W_up + b_up)
  const float* const u = s_z + 3 * Hkv;
  const int HD = Hq * D;
  for (int col = tid; col < HD; col += NT) {
    float z = a.b_up ? a.b_up[col] : 0.0f;
    for (int q = 0; q < a.r; ++q) z = fmaf(u[q], load_elem<BF16>(a.W_up, (int64_t)q * HD + col), z);
    w.gam[(int64_t)b * HD + col] = sigmoid(z);
  }
  // ---- per KV head (one wave each): the stored key (L2-normalised, rotated,
  // rounded like the cache), then for each of its G query heads the rotated
  // query and the token's logit against its own key (log2 units)
  const float qs2 = a.scale * kLog2e;
  for (int h = wv; h < Hkv; h += NT / 64) {
    const int s = b * Hkv + h;
    float k0 = 0.0f, k1 = 0.0f;
    if (lane < HALF) {
      k0 = load_elem<BF16>(a.k, (int64_t)s * D + lane);
      k1 = load_elem<BF16>(a.k, (int64_t)s * D + lane + HALF);
    }
    const float inv = 1.0f / fmaxf(sqrtf(wave_sum(k0 * k0 + k1 * k1)), 1e-12f);
    float r0 = 0.0f, r1 = 0.0f;
    if (lane < HALF) {
      const float n0 = k0 * inv, n1 = k1 * inv;
      r0 = fmaf(n0, s_cs[lane], -n1 * s_sn[lane]);
      r1 = fmaf(n1, s_cs[lane], n0 * s_sn[lane]);
      if constexpr (BF16) {
        r0 = bf16_to_f32(f32_to_bf16(r0));
        r1 = bf16_to_f32(f32_to_bf16(r1));
      }
      w.tkey[(int64_t)s * D + lane] = r0;
      w.tkey[(int64_t)s * D + lane + HALF] = r1;
    }
    for (int g = 0; g < G; ++g) {
      const int hq = h * G + g;
      const int64_t qi = ((int64_t)b * Hq + hq) * D + lane;
      float e = 0.0f;
      if (lane < HALF) {
        const float q0 = load_elem<BF16>(a.q, qi), q1 = load_elem<BF16>(a.q, qi + HALF);
        const float t0 = fmaf(q0, s_cs[lane], -q1 * s_sn[lane]);
        const float t1 = fmaf(q1, s_cs[lane], q0 * s_sn[lane]);
        w.tq[qi] = t0;
        w.tq[qi + HALF] = t1;
        e = fmaf(t0, r0, t1 * r1);
      }
      e = wave_sum(e);
      if (lane == 0) w.es[(int64_t)b * Hq + hq] = e * qs2;
    }
  }
}

// ---------------------------------------------------------------------------
// launch 2: the tiles
// ---------------------------------------------------------------------------
template <int D, int G, bool BF16, bool COMPACT>
__global__ __launch_bounds__(kTileThreads) void decode_tile_kernel(DecodeKArgs karg) {
  const DecodeKArgs& K = *(const DecodeKArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const LayerArgs& a = K.a;
  const DecodeWs& w = K.w;
  using Sh = TileShape<D, decode_nb(D, G)>;
  constexpr int LPE = Sh::LPE, NGW = Sh::NGW, NB = Sh::NB, TW = Sh::TW, TWG = Sh::TWG;
  constexpr int NT = kTileThreads;
  constexpr int OPT = (G * D + NT - 1) / NT;  // outputs (g, i) per thread
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  __shared__ int s_kt;
  __shared__ int s_flag;
  __shared__ int s_pre;
  __shared__ int s_cnt[kTileWaves];
  __shared__ float s_tp[kTileWaves][NGW * D];                   // per-wave transpose of the weighted V
  __shared__ float s_po[kTileWaves * G * D];                    // wave partials: weighted V
  __shared__ float s_pm[kTileWaves * G], s_pl[kTileWaves * G];  // wave partials: max (log2), sum

  if ((int)blockIdx.x >= *w.ntiles) return;  // past this step's tiles
  const int4 m0 = w.map[2 * blockIdx.x + 0];
  const int4 m1 = w.map[2 * blockIdx.x + 1];
  const int seg = m0.x;
  const int len = m0.z;
  const int ntile = m0.w;
  const int pbase = m1.x;  // record number of the segment's first tile
  const int64_t off = (int64_t)(uint32_t)m1.y | ((int64_t)m1.z << 32);
  const bool single = ntile == 1;
  int kt = 0;
  if (!single) {  // tile numbers in arrival order: a tile's predecessors have started
    if (tid == 0) s_kt = add_coh(&w.segtk[seg], 1);
    __syncthreads();
    kt = s_kt;
  }
  const int Hkv = a.H_kv;
  const int b = seg / Hkv;
  const int h = seg - b * Hkv;
  const int grp = lane / LPE;
  const int c = lane - grp * LPE;
  const int e0 = kt * TWG + wv * TW + grp * NB;

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
  // ---- the token: rotated queries of the group and the stored key (8 dims
  // per lane), the query/similarity part of the pair term
  float qv[G][8], ktv[8];
  {
    const float* qrow = w.tq + ((int64_t)b * a.H_q + h * G) * D + 8 * c;
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
  const float row2 = w.tokf[2 * seg];
  const float tau = K.tau;
  const float qs2 = a.scale * kLog2e;
  const PairCoef pc = pair_coef(a.terms);
  const float kscale = (a.terms & 2) ? pc.inv_n2 : 0.0f;

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
      s_po[(wv * G + g) * D + half * 64 + lane] = sum;
    }
    __builtin_amdgcn_wave_barrier();  // the next head reuses the scratch
    if (lane == 0) {
      s_pm[wv * G + g] = ms[g];
      s_pl[wv * G + g] = l;
    }
  }
  __syncthreads();  // partials and live counts in LDS; every row of the tile is in registers

  int count = 0, wbase = 0;
  if constexpr (COMPACT) {
#pragma unroll
    for (int w2 = 0; w2 < kTileWaves; ++w2) {
      wbase += (w2 < wv) ? s_cnt[w2] : 0;
      count += s_cnt[w2];
    }
    // this tile's count (the first tile's is already its inclusive prefix)
    if (!single && tid == 0)
      st64_coh(&K.ctl.dec_state[pbase + kt], (unsigned long long)((count << 2) | (kt == 0 ? 2 : 1)));
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
    for (int w2 = 0; w2 < kTileWaves; ++w2) M = fmaxf(M, s_pm[w2 * G + g]);
    const float Ms = (M == kNegInf) ? 0.0f : M;
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < kTileWaves; ++w2) {
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
    const int64_t prow = (int64_t)(pbase + kt);
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
    }
  }

  // ---- combine: the token's own term, the output gate, y
  if (combines) {
    const int Hq = a.H_q;
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int idx = u * NT + tid;
      if (idx < G * D) {
        const int g = idx / D;
        const int i = idx - g * D;
        const int col = (h * G) * D + idx;
        const float es = w.es[(int64_t)b * Hq + h * G + g];
        const float vn = elem_at<BF16>(reinterpret_cast<const char*>(a.v), (uint32_t)((seg * D + i) * EB));
        const float M = fmaxf(Mo[u], es);
        const float rs = __builtin_amdgcn_exp2f(Mo[u] - M);  // Mo = -inf gives 0
        const float pe = __builtin_amdgcn_exp2f(es - M);
        const float L = fmaf(Lo[u], rs, pe);
        const float O = fmaf(Oo[u], rs, pe * vn);
        const int64_t yo = (int64_t)b * Hq * D + col;
        const float yv = w.gam[yo] * (O / L);
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
    if (single || kt == 0) {
      if (tid == 0) s_pre = 0;
    } else if (wv == 0) {
      const unsigned long long* st = K.ctl.dec_state + pbase;
      int prefix = 0;
      int cpos = kt - 1;  // next predecessor to examine
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
          if (lane == 0) atomicOr(a.status, 2);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0) {
        st64_coh(&K.ctl.dec_state[pbase + kt], (unsigned long long)(((prefix + count) << 2) | 2));
        s_pre = prefix;
      }
    }
    __syncthreads();
    // ---- the survivors, in order; rows already in place are not rewritten
    const int P = s_pre;
    int32_t* const kept = K.kept;
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

  // ---- the new entry: the segment's last tile after the survivors when
  // compacting, else the first tile at the old length; then the new length
  const bool appends = COMPACT ? (kt == ntile - 1) : (kt == 0);
  if (appends) {
    const bool room = len < a.seg_cap[seg];
    if (room && tid < D) {
      const int64_t dst = (off + npos) * D + tid;
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
        a.lam[off + npos] = 0.0f;
        a.lk[off + npos] = w.tokf[2 * seg + 1];
        if (COMPACT && K.kept) K.kept[off + npos] = len;
      } else {
        atomicOr(a.status, 1);
      }
      a.seg_len[seg] = room ? npos + 1 : npos;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int tile_entries(int d, int nb) { return (64 / (d / 8)) * nb * kTileWaves; }

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
  int* segtk = reinterpret_cast<int*>(take(sizeof(int) * S));
  int* ntiles = reinterpret_cast<int*>(take(sizeof(int)));
  int4* map = reinterpret_cast<int4*>(take(sizeof(int4) * 2 * mt));
  float* tq = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q * a.d));
  float* tkey = reinterpret_cast<float*>(take(sizeof(float) * S * a.d));
  float* gam = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q * a.d));
  float* tokf = reinterpret_cast<float*>(take(sizeof(float) * S * 2));
  float* es = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q));
  float* part_o = reinterpret_cast<float*>(take(sizeof(float) * mt * G * a.d));
  float* part_ml = reinterpret_cast<float*>(take(sizeof(float) * mt * G * 2));
  if (w) {
    w->segtk = segtk;
    w->ntiles = ntiles;
    w->map = map;
    w->tq = tq;
    w->tkey = tkey;
    w->gam = gam;
    w->tokf = tokf;
    w->es = es;
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
  const int twg = TileShape<D, decode_nb(D, G)>::TWG;
  const DecodeKArgs k{a, w, ctl, tau, kept, twg};
  hipLaunchKernelGGL((decode_token_kernel<D, BF16>), dim3(a.B + 1), dim3(kTokThreads), 0, st, k);
  const int64_t mt = decode_max_tiles(a, twg);
  if (mt > (1 << 30)) return hipErrorInvalidValue;
  const int grid = (int)mt;
  if (compact) {
    hipLaunchKernelGGL((decode_tile_kernel<D, G, BF16, true>), dim3(grid), dim3(kTileThreads), 0, st, k);
  } else {
    hipLaunchKernelGGL((decode_tile_kernel<D, G, BF16, false>), dim3(grid), dim3(kTileThreads), 0, st, k);
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
