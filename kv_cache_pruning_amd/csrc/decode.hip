// UA decode step on a ragged, per-KV-head pruned cache (gfx950): two kernels.
//
// 1. decode_token_kernel, grid (B, head splits): everything that depends only
//    on the new token -- gate projections x W_dec + b_dec and x W_dn (one
//    vectorised pass over the rows of both matrices), log-sigmoid gates,
//    RoPE of the queries and of the L2-normalised key (angles in fp64), the
//    key rounded to the cache type, the output gate sigmoid(u W_up + b_up),
//    the new token's own logit, and the cache append.  ("A Self-Pruning
//    Transformer ...", ai4snews Figure 1 caption: L2-normalised keys, RoPE,
//    low-rank sigmoid output gate.)
// 2. decode_main_kernel: one workgroup per tile of a segment (segment = one
//    sequence and KV head), mapped from the read-only capacities so that no
//    workgroup depends on a length another one updates.  Each cached entry is
//    read once: its key row feeds <q~_g, k~_j> for the G query heads and
//    <k~_t, k~_j> for the similarity term; the pair term (geometric mean of
//    the enabled decays in log space, paperlayer.ai sections 4 and 4.1) is
//    added to the log-bias in place; entries below log p drop out of the step
//    (section 4.2); an online-softmax partial (max, sum, weighted V) is
//    written per tile.  The last tile of a segment to arrive merges the
//    partials with the new token's own term, applies the gate and advances
//    the segment length.
//
// Cross-workgroup data use relaxed agent-scope atomic loads/stores (coherent
// across the XCDs without cache-wide write-back or invalidation).  The
// arrival counters live in the workspace control block and return to zero at
// the end of every call.
//
// Lane layout of the entry loop: a wave splits into groups of LPE = d/8
// lanes; lane c of a group holds dims [8c, 8c+8) of one entry at a time, so a
// group's 16-byte (bf16) row loads are contiguous.  Each group walks NB
// consecutive entries; dot products are reduced inside the group with DPP.

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

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// 1. token kernel
// ---------------------------------------------------------------------------
constexpr int kTokThreads = 512;  // all threads load; per-output work uses the first 256
constexpr int kTokOut = 256;

// Element e of a bf16 / fp32 row held as raw 16-byte chunks.
template <bool BF16>
__device__ __forceinline__ float chunk_elem(const u32x4& c, int t) {
  if constexpr (BF16) {
    const uint32_t wd = t < 2 ? c.x : (t < 4 ? c.y : (t < 6 ? c.z : c.w));
    return (t & 1) ? bf16_hi(wd) : bf16_lo(wd);
  } else {
    return __uint_as_float(t == 0 ? c.x : (t == 1 ? c.y : (t == 2 ? c.z : c.w)));
  }
}

template <bool BF16>
__global__ __launch_bounds__(kTokThreads) void decode_token_kernel(LayerArgs a, DecodeWs w) {
  constexpr int CW = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int b = blockIdx.x;
  const int sp = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int D = a.d;
  const int half = D >> 1;
  const int Hkv = a.H_kv;
  const int Hq = a.H_q;
  const int G = Hq / Hkv;
  const int Dm = a.D_model;
  const int r = a.r;
  const int HP = kTokOut / D;  // query heads per split
  const int a0 = sp * HP;
  const int a1 = min(Hq, a0 + HP);
  const int h0 = a0 / G;        // KV heads this split touches: h0..h1
  const int h1 = (a1 - 1) / G;
  const int hown = (h0 * G >= a0) ? h0 : h0 + 1;  // first KV head it owns
  const int nown = h1 - hown + 1;                 // owned KV heads (0..4)
  const int ncol = 3 * nown;                      // gate columns it needs

  __shared__ float s_z[12];
  __shared__ float s_u[kMaxRank];
  __shared__ float s_cos[64], s_sin[64];
  __shared__ float s_q[kTokOut];
  __shared__ float s_kt[4][128];
  __shared__ uint16_t s_kb[4][128];

  const int pos = a.next_pos[b];
  const int64_t xb = (int64_t)b * Dm;

  // =================== issue the loads ===================
  // Every load below is unconditional from an index clamped into range, and
  // masking happens where the values are used: a load whose result feeds a
  // select right away makes the compiler wait for it before the next load.
  //
  // x W_dec and x W_dn in one pass over rows of [W_dec | W_dn] cut into
  // 16-byte chunks (nzc chunks of W_dec, nuc of W_dn), padded to a power of
  // two so that each thread owns one chunk column; rows are split over the
  // threads sharing it.
  const int nzc = (3 * Hkv + CW - 1) / CW;
  const int nuc = (r + CW - 1) / CW;
  int ncp = 1;
  while (ncp < nzc + nuc) ncp <<= 1;  // <= 32
  const int kc = tid & (ncp - 1);
  const int rstep = kTokThreads / ncp;
  const bool vec = ((3 * Hkv) % CW == 0) && (r % CW == 0);
  const bool own_dec = kc < nzc;
  const bool own_dn = !own_dec && kc < nzc + nuc;
  const char* mbase = own_dec ? reinterpret_cast<const char*>(a.W_dec) : reinterpret_cast<const char*>(a.W_dn);
  const int mcols = own_dec ? 3 * Hkv : r;
  const int mc0 = (own_dec ? kc : (own_dn ? kc - nzc : 0)) * CW;
  constexpr int kRows = 32;  // rows per thread per pass (one round trip)
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  // query element of this thread and its rotation partner
  const int qh = a0 + tid / D, qi = tid % D;
  const int64_t qbase = ((int64_t)b * Hq + min(qh, Hq - 1)) * D;
  const float qx = load_elem<BF16>(a.q, qbase + qi);
  const float qp = load_elem<BF16>(a.q, qbase + (qi < half ? qi + half : qi - half));
  // key elements (wave per touched KV head)
  const int64_t kbase = ((int64_t)b * Hkv + min(h0 + wv, Hkv - 1)) * D;
  const float kx0 = load_elem<BF16>(a.k, kbase + (lane & (half - 1)));
  const float kx1 = load_elem<BF16>(a.k, kbase + (lane & (half - 1)) + half);
  // output-gate weights of this thread's column
  constexpr int kUpRows = 16;
  float up[kUpRows];
  const bool uown = tid < kTokOut && a0 + tid / D < a1;
  const int ucol = a0 * D + tid;
  const int ucc = uown ? ucol : 0;
#pragma unroll
  for (int c = 0; c < kUpRows; ++c) up[c] = load_elem<BF16>(a.W_up, (int64_t)min(c, r - 1) * Hq * D + ucc);

  // =================== RoPE table while the loads fly ===================
  if (tid < half) {
    double sn, cs;
    sincos((double)pos * a.inv_freq[tid], &sn, &cs);
    s_cos[tid] = (float)cs;
    s_sin[tid] = (float)sn;
  }

  float acc[CW];
#pragma unroll
  for (int t = 0; t < CW; ++t) acc[t] = 0.0f;
  for (int i0 = tid / ncp; i0 < Dm; i0 += kRows * rstep) {
    u32x4 raw[kRows];
    float xr[kRows];
#pragma unroll
    for (int q = 0; q < kRows; ++q) {
      const int i = min(i0 + q * rstep, Dm - 1);
      xr[q] = load_elem<BF16>(a.x, xb + i);
      raw[q] = vec ? *reinterpret_cast<const u32x4*>(mbase + ((int64_t)i * mcols + mc0) * (BF16 ? 2 : 4)) : zero4;
    }
    const bool mine = own_dec || own_dn;
#pragma unroll
    for (int q = 0; q < kRows; ++q) {
      const int i = i0 + q * rstep;
      const float xi = (mine && i < Dm) ? xr[q] : 0.0f;
      if (vec) {
#pragma unroll
        for (int t = 0; t < CW; ++t) acc[t] = fmaf(xi, chunk_elem<BF16>(raw[q], t), acc[t]);
      } else if (xi != 0.0f) {  // rows not 16-byte aligned: element loads
#pragma unroll
        for (int t = 0; t < CW; ++t)
          if (mc0 + t < mcols)
            acc[t] = fmaf(xi, load_elem<BF16>(mbase == reinterpret_cast<const char*>(a.W_dec) ? a.W_dec : a.W_dn,
                                              (int64_t)i * mcols + mc0 + t), acc[t]);
      }
    }
  }
  // reduce over the threads owning the same chunk column: lanes kc, kc+ncp, ..., then waves
#pragma unroll
  for (int t = 0; t < CW; ++t) {
    float v = acc[t];
    for (int o = ncp; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    acc[t] = v;
  }
  __shared__ float s_zu[kTokThreads / 64][32 * 8];
  if (lane < ncp) {
#pragma unroll
    for (int t = 0; t < CW; ++t) s_zu[wv][lane * CW + t] = acc[t];
  }
  __syncthreads();
  if (tid < (nzc + nuc) * CW) {
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < kTokThreads / 64; ++q) sum += s_zu[q][tid];
    const int kk = tid / CW, col = tid % CW + (kk < nzc ? kk : kk - nzc) * CW;
    if (kk < nzc) {
      // pre-activation of gate column col; keep the owned heads' ones
      if (col < 3 * Hkv) {
        const int m = col / Hkv, h = col - m * Hkv;
        if (h >= hown && h < hown + nown) s_z[3 * (h - hown) + m] = sum + a.b_dec[col];
      }
    } else if (col < r) {
      s_u[col] = sum;
    }
  }
  __syncthreads();

  // =================== rotated queries and keys ===================
  if (tid < kTokOut && qh < a1) {
    const float out = (qi < half) ? fmaf(qx, s_cos[qi], -qp * s_sin[qi]) : fmaf(qx, s_cos[qi - half], qp * s_sin[qi - half]);
    s_q[tid] = out;
    w.qt[((int64_t)b * Hq + qh) * D + qi] = out;
  }
  if (wv <= h1 - h0) {
    const int h = h0 + wv;
    const int s = b * Hkv + h;
    const int64_t kb = (int64_t)s * D;
    float k0 = (lane < half) ? kx0 : 0.0f;
    float k1 = (lane < half) ? kx1 : 0.0f;
    const float inv = 1.0f / fmaxf(sqrtf(wave_sum(k0 * k0 + k1 * k1)), 1e-12f);
    k0 *= inv;
    k1 *= inv;
    if (lane < half) {
      float r0 = fmaf(k0, s_cos[lane], -k1 * s_sin[lane]);
      float r1 = fmaf(k1, s_cos[lane], k0 * s_sin[lane]);
      uint16_t b0 = 0, b1 = 0;
      if constexpr (BF16) {
        b0 = f32_to_bf16(r0);
        b1 = f32_to_bf16(r1);
        r0 = bf16_to_f32(b0);
        r1 = bf16_to_f32(b1);
      }
      s_kt[wv][lane] = r0;
      s_kt[wv][lane + half] = r1;
      s_kb[wv][lane] = b0;
      s_kb[wv][lane + half] = b1;
    }
    // the split that holds query head h*G owns KV head h: gates, stored key, append
    if (h >= hown) {
      const int len = a.seg_len[s];
      const int cap = a.seg_cap[s];
      const int64_t off = a.seg_off[s];
      if (lane < half) {
        w.kt[kb + lane] = s_kt[wv][lane];
        w.kt[kb + lane + half] = s_kt[wv][lane + half];
      }
      if (len < cap && lane < half) {
        const int64_t dst = (off + len) * D;
        if constexpr (BF16) {
          uint16_t* K = reinterpret_cast<uint16_t*>(a.K);
          uint16_t* V = reinterpret_cast<uint16_t*>(a.V);
          const uint16_t* vin = reinterpret_cast<const uint16_t*>(a.v);
          K[dst + lane] = s_kb[wv][lane];
          K[dst + lane + half] = s_kb[wv][lane + half];
          V[dst + lane] = vin[kb + lane];
          V[dst + lane + half] = vin[kb + lane + half];
        } else {
          float* K = reinterpret_cast<float*>(a.K);
          float* V = reinterpret_cast<float*>(a.V);
          const float* vin = reinterpret_cast<const float*>(a.v);
          K[dst + lane] = s_kt[wv][lane];
          K[dst + lane + half] = s_kt[wv][lane + half];
          V[dst + lane] = vin[kb + lane];
          V[dst + lane + half] = vin[kb + lane + half];
        }
      }
      if (lane == 0) {
        const int jz = 3 * (h - hown);
        const float lq = log_sigmoid(s_z[jz + 0]);
        const float lkk = log_sigmoid(s_z[jz + 1]);
        const float lb = log_sigmoid(s_z[jz + 2]);
        w.gates[s * 4 + 0] = lq;
        w.gates[s * 4 + 1] = lkk;
        w.gates[s * 4 + 2] = lb;
        w.gates[s * 4 + 3] = 0.0f;
        w.len_old[s] = len;
        if (len < cap) {
          a.lam[off + len] = 0.0f;
          a.lk[off + len] = lkk;
        } else {
          atomicOr(a.status, 1);
        }
      }
    }
  }
  __syncthreads();

  // =================== own logits and output gate ===================
  if (wv < a1 - a0) {  // one wave per query head of the split
    const int hw = (a0 + wv) / G - h0;
    float acc = 0.0f;
    for (int i = lane; i < D; i += 64) acc = fmaf(s_q[wv * D + i], s_kt[hw][i], acc);
    acc = wave_sum(acc);
    if (lane == 0) w.eself[b * Hq + a0 + wv] = acc * a.scale * kLog2e;
  }
  if (uown) {
    float gsum = a.b_up ? a.b_up[ucol] : 0.0f;
#pragma unroll
    for (int c = 0; c < kUpRows; ++c)
      if (c < r) gsum = fmaf(s_u[c], up[c], gsum);  // rows >= r were clamped loads
    for (int c = kUpRows; c < r; ++c) gsum = fmaf(s_u[c], load_elem<BF16>(a.W_up, (int64_t)c * Hq * D + ucol), gsum);
    w.gamma[(int64_t)b * Hq * D + ucol] = sigmoid(gsum);
  }

  // ---- the last split of this sequence advances its position
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0 && add_coh(&w.cntb[b], 1) == (int)gridDim.y - 1) {
    a.next_pos[b] = pos + 1;
    sti_coh(&w.cntb[b], 0);
  }
}

// ---------------------------------------------------------------------------
// 2. main kernel
// ---------------------------------------------------------------------------
template <bool BF16>
struct Row8 {
  u32x4 w[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ void row_load(Row8<BF16>& r, const void* base, int64_t elem) {
  if constexpr (BF16) {
    r.w[0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem);
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(base) + elem);
    r.w[0] = p[0];
    r.w[1] = p[1];
  }
}

template <bool BF16>
__device__ __forceinline__ void row_f32(const Row8<BF16>& r, float (&o)[8]) {
  if constexpr (BF16) {
    o[0] = bf16_lo(r.w[0].x); o[1] = bf16_hi(r.w[0].x);
    o[2] = bf16_lo(r.w[0].y); o[3] = bf16_hi(r.w[0].y);
    o[4] = bf16_lo(r.w[0].z); o[5] = bf16_hi(r.w[0].z);
    o[6] = bf16_lo(r.w[0].w); o[7] = bf16_hi(r.w[0].w);
  } else {
    o[0] = __uint_as_float(r.w[0].x); o[1] = __uint_as_float(r.w[0].y);
    o[2] = __uint_as_float(r.w[0].z); o[3] = __uint_as_float(r.w[0].w);
    o[4] = __uint_as_float(r.w[1].x); o[5] = __uint_as_float(r.w[1].y);
    o[6] = __uint_as_float(r.w[1].z); o[7] = __uint_as_float(r.w[1].w);
  }
}

template <int D>
struct DecodeShape {
  static constexpr int LPE = D / 8;       // lanes per entry
  static constexpr int NGW = 64 / LPE;    // entry groups per wave
  static constexpr int NB = 4;            // entries per group
  static constexpr int TW = NGW * NB;     // entries per wave
  static constexpr int NWAVE = 4;
  static constexpr int NT = 64 * NWAVE;
  static constexpr int TWG = TW * NWAVE;  // entries per workgroup tile
  static constexpr int NP = NGW * NWAVE;  // partials per workgroup
};

__device__ __forceinline__ int tiles_of(int n, int twg) { return n <= 0 ? 1 : ceil_div(n, twg); }

template <int D, int G, bool BF16>
__global__ __launch_bounds__(DecodeShape<D>::NT) void decode_main_kernel(LayerArgs a, DecodeWs w, float tau) {
  using Sh = DecodeShape<D>;
  constexpr int LPE = Sh::LPE, NGW = Sh::NGW, NB = Sh::NB, TW = Sh::TW, NT = Sh::NT, TWG = Sh::TWG, NP = Sh::NP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int S = a.B * a.H_kv;
  const int Hkv = a.H_kv;

  __shared__ int s_scan[NT / 64 + 1];
  __shared__ int s_info[4];
  __shared__ int s_last;
  __shared__ float s_po[NP * G * D];
  __shared__ float s_pm[NP * G];
  __shared__ float s_pl[NP * G];

  // ---- (segment, tile) from the read-only capacities
  {
    const int per = (S + NT - 1) / NT;
    const int sb = tid * per;
    const int se = min(S, sb + per);
    int mine = 0;
    for (int s = sb; s < se; ++s) mine += tiles_of(w.len_old[s], TWG);
    int total;
    const int excl = block_exclusive_scan<NT>(mine, s_scan, &total);
    if ((int)blockIdx.x >= total) return;
    int run = excl;
    for (int s = sb; s < se; ++s) {
      const int nt = tiles_of(w.len_old[s], TWG);
      if ((int)blockIdx.x >= run && (int)blockIdx.x < run + nt) {
        s_info[0] = s;
        s_info[1] = blockIdx.x - run;
        s_info[2] = nt;
        s_info[3] = run;
      }
      run += nt;
    }
    __syncthreads();
  }
  const int seg = s_info[0];
  const int kt_ = s_info[1];
  const int ntile = s_info[2];  // tiles of this segment (all arrive)
  const int pbase = s_info[3];  // first partial row of this segment
  const int b = seg / Hkv;
  const int h = seg - b * Hkv;
  const int len = w.len_old[seg];  // length before this step's append
  const int cap = a.seg_cap[seg];
  const int64_t off = a.seg_off[seg];
  const float qs2 = a.scale * kLog2e;

  {
    const int grp = lane / LPE;
    const int c = lane - grp * LPE;
    const int e0 = kt_ * TWG + wv * TW + grp * NB;

    // ---- cached entries: issue every load first
    Row8<BF16> kr[NB], vr[NB];
    float lamv[NB], lkv[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int j = e0 + bb;
      if (j < len) {
        row_load<BF16>(kr[bb], a.K, (off + j) * D + 8 * c);
        row_load<BF16>(vr[bb], a.V, (off + j) * D + 8 * c);
        lamv[bb] = a.lam[off + j];
        lkv[bb] = a.lk[off + j];
      } else {
        lamv[bb] = kNegInf;
        lkv[bb] = 0.0f;
#pragma unroll
        for (int t = 0; t < (BF16 ? 1 : 2); ++t) kr[bb].w[t] = vr[bb].w[t] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    // ---- token-side data (written by the token kernel)
    float qv[G][8];
    float ktv[8];
#pragma unroll
    for (int g = 0; g < G; ++g) load8<false>(w.qt, ((int64_t)b * a.H_q + h * G + g) * D + 8 * c, qv[g]);
    load8<false>(w.kt, (int64_t)seg * D + 8 * c, ktv);
    const PairCoef pc = pair_coef(a.terms);
    const float lq = w.gates[seg * 4 + 0];
    const float lb = w.gates[seg * 4 + 2];
    const float row2 = (((a.terms & 1) ? lq : 0.0f) + ((a.terms & 4) ? lb : 0.0f)) * pc.inv_n2;
    const float kscale = (a.terms & 2) ? pc.inv_n2 : 0.0f;

    // ---- dot products, pair term, bias update, logits
    float e2[G][NB];
    float newlam[NB];
    bool changed[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
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
      const float l0 = lamv[bb];
      const bool valid = e0 + bb < len;
      const bool alive = valid && (l0 >= tau);
      const float A = pair_A(pc, row2, lkv[bb] * kscale, ps);
      const float l1 = alive ? l0 + A : l0;
      const bool live = alive && (l1 >= tau);
      newlam[bb] = l1;
      changed[bb] = alive;
      const float lb2 = l1 * kLog2e;
#pragma unroll
      for (int g = 0; g < G; ++g) e2[g][bb] = live ? fmaf(pq[g], qs2, lb2) : kNegInf;
    }
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

    // ---- group partials -> LDS
    const int pidx = wv * NGW + grp;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = e2[g][0];
#pragma unroll
      for (int bb = 1; bb < NB; ++bb) m = fmaxf(m, e2[g][bb]);
      const float ms = (m == kNegInf) ? 0.0f : m;
      float l = 0.0f;
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = 0.0f;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const float p = __builtin_amdgcn_exp2f(e2[g][bb] - ms);
        l += p;
        float vf[8];
        row_f32<BF16>(vr[bb], vf);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = fmaf(p, vf[i], o[i]);
      }
      float4* dst = reinterpret_cast<float4*>(s_po + (pidx * G + g) * D + 8 * c);
      dst[0] = make_float4(o[0], o[1], o[2], o[3]);
      dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      if (c == 0) {
        s_pm[pidx * G + g] = m;
        s_pl[pidx * G + g] = l;
      }
    }
    __syncthreads();

    // ---- merge the workgroup's partials -> workspace row pbase + kt_
    const int64_t prow = (int64_t)(pbase + kt_);
    for (int idx = tid; idx < G * D; idx += NT) {
      const int g = idx / D;
      const int i = idx - g * D;
      float M = kNegInf;
#pragma unroll
      for (int p = 0; p < NP; ++p) M = fmaxf(M, s_pm[p * G + g]);
      const float Ms = (M == kNegInf) ? 0.0f : M;
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float wgt = __builtin_amdgcn_exp2f(s_pm[p * G + g] - Ms);
        L = fmaf(s_pl[p * G + g], wgt, L);
        O = fmaf(s_po[(p * G + g) * D + i], wgt, O);
      }
      st_coh(w.part_o + (prow * G + g) * D + i, O);
      if (i == 0) {
        st_coh(w.part_ml + (prow * G + g) * 2 + 0, M);
        st_coh(w.part_ml + (prow * G + g) * 2 + 1, L);
      }
    }
  }

  // ---- arrival; the last workgroup of the segment combines
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_last = (add_coh(&w.cnt[seg], 1) == ntile - 1);
  __syncthreads();
  if (!s_last) return;

  // running merge state per output (g, i): the new token's own term first
  constexpr int OPT = (G * D + NT - 1) / NT;
  float Mr[OPT], Lr[OPT], Or[OPT];
#pragma unroll
  for (int u = 0; u < OPT; ++u) {
    const int idx = u * NT + tid;
    if (idx < G * D) {
      const int g = idx / D;
      const int i = idx - g * D;
      Mr[u] = w.eself[b * a.H_q + h * G + g];
      Lr[u] = 1.0f;
      Or[u] = load_elem<BF16>(a.v, (int64_t)seg * D + i);
    }
  }
  constexpr int TC = 32;           // tiles per pass
  float* s_cm = s_po;              // [G][TC] tile maxima
  float* s_cl = s_po + G * TC;     // [G][TC] tile sums
  for (int p0 = 0; p0 < ntile; p0 += TC) {
    const int np = min(TC, ntile - p0);
    __syncthreads();
    for (int idx = tid; idx < G * TC; idx += NT) {
      const int g = idx / TC;
      const int p = idx - g * TC;
      if (p < np) {
        const int64_t pr = (int64_t)(pbase + p0 + p);
        s_cm[idx] = ld_coh(w.part_ml + (pr * G + g) * 2 + 0);
        s_cl[idx] = ld_coh(w.part_ml + (pr * G + g) * 2 + 1);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int idx = u * NT + tid;
      if (idx < G * D) {
        const int g = idx / D;
        const int i = idx - g * D;
        float M = Mr[u];
        for (int p = 0; p < np; ++p) M = fmaxf(M, s_cm[g * TC + p]);
        const float rs = __builtin_amdgcn_exp2f(Mr[u] - M);
        float L = Lr[u] * rs, O = Or[u] * rs;
        float po[TC];
#pragma unroll
        for (int p = 0; p < TC; ++p)
          po[p] = (p < np) ? ld_coh(w.part_o + ((int64_t)(pbase + p0 + p) * G + g) * D + i) : 0.0f;
#pragma unroll
        for (int p = 0; p < TC; ++p) {
          if (p < np) {
            const float wgt = __builtin_amdgcn_exp2f(s_cm[g * TC + p] - M);
            L = fmaf(s_cl[g * TC + p], wgt, L);
            O = fmaf(po[p], wgt, O);
          }
        }
        Mr[u] = M;
        Lr[u] = L;
        Or[u] = O;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < OPT; ++u) {
    const int idx = u * NT + tid;
    if (idx < G * D) {
      const int g = idx / D;
      const int i = idx - g * D;
      const int64_t yo = ((int64_t)b * a.H_q + h * G + g) * D + i;
      const float yv = w.gamma[yo] * (Or[u] / Lr[u]);
      if (a.y_bf16) {
        reinterpret_cast<uint16_t*>(a.y)[yo] = f32_to_bf16(yv);
      } else {
        reinterpret_cast<float*>(a.y)[yo] = yv;
      }
    }
  }
  if (tid == 0) {
    a.seg_len[seg] = len < cap ? len + 1 : len;
    sti_coh(&w.cnt[seg], 0);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int decode_tile_entries(int d) { return d == 64 ? DecodeShape<64>::TWG : DecodeShape<128>::TWG; }

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
  float* qt = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q * a.d));
  float* kt = reinterpret_cast<float*>(take(sizeof(float) * S * a.d));
  float* gates = reinterpret_cast<float*>(take(sizeof(float) * S * 4));
  int* len_old = reinterpret_cast<int*>(take(sizeof(int) * S));
  float* eself = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q));
  float* gamma = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q * a.d));
  float* part_o = reinterpret_cast<float*>(take(sizeof(float) * mt * G * a.d));
  float* part_ml = reinterpret_cast<float*>(take(sizeof(float) * mt * G * 2));
  if (w) {
    w->qt = qt;
    w->kt = kt;
    w->gates = gates;
    w->len_old = len_old;
    w->eself = eself;
    w->gamma = gamma;
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
  w.cntb = ctl.dec_cntb;
  return w;
}

template <int D, int G, bool BF16>
static hipError_t launch_main(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st) {
  using Sh = DecodeShape<D>;
  hipLaunchKernelGGL((decode_main_kernel<D, G, BF16>), dim3(w.max_tiles), dim3(Sh::NT), 0, st, a, w, tau);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_main_g(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st) {
  switch (a.H_q / a.H_kv) {
    case 1: return launch_main<D, 1, BF16>(a, w, tau, st);
    case 2: return launch_main<D, 2, BF16>(a, w, tau, st);
    case 3: return launch_main<D, 3, BF16>(a, w, tau, st);
    case 4: return launch_main<D, 4, BF16>(a, w, tau, st);
    case 8: return launch_main<D, 8, BF16>(a, w, tau, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const LayerArgs& a, const DecodeWs& w, float tau, hipStream_t st) {
  const int splits = (a.H_q * a.d + kTokOut - 1) / kTokOut;
  if (a.bf16) {
    hipLaunchKernelGGL((decode_token_kernel<true>), dim3(a.B, splits), dim3(kTokThreads), 0, st, a, w);
  } else {
    hipLaunchKernelGGL((decode_token_kernel<false>), dim3(a.B, splits), dim3(kTokThreads), 0, st, a, w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.d == 64) return a.bf16 ? launch_main_g<64, true>(a, w, tau, st) : launch_main_g<64, false>(a, w, tau, st);
  return a.bf16 ? launch_main_g<128, true>(a, w, tau, st) : launch_main_g<128, false>(a, w, tau, st);
}

}  // namespace ua
