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
// Workgroups take ids from an atomic ticket, so every wait below is on a
// workgroup that started earlier.
//  * ids [0, B*NS): per-token work of sequence b = id / NS, split NS ways over
//    the query heads (NS = H_q d / 256): a slice of the rows of
//    x [W_dec | W_dn] (partial sums, reduced by their consumers), the rotated
//    queries of the split's heads, the stored key of its KV heads and the
//    token's own logits.  The last step publishes a per-sequence counter.
//  * later ids: one tile of TWG entries of one segment (segment = sequence and
//    KV head), mapped from the segment lengths, which stay constant until the
//    kernel ends.  The tile issues its cache loads, waits for its sequence's
//    token data, and reads each entry once: the key row feeds the G query
//    dot products and the key-similarity dot product, the pair term updates
//    the log-bias, and an online-softmax partial (max, sum, weighted V) goes
//    to the workspace.  With COMPACT the surviving entries then move down in
//    place: the tile publishes its live count, looks back over the earlier
//    tiles of its segment for its destination (decoupled look-back, up to 64
//    predecessors per wave step), waits until every earlier tile whose rows
//    it overwrites holds its own rows in registers, and stores.  Without
//    COMPACT the updated log-biases are written in place.
//  * The last tile of a segment to arrive merges the partials with the
//    token's own term, forms the output gate for its query heads from its
//    slice of W_up, writes y and appends the new entry (after the survivors
//    when compacting).  The last workgroup overall commits the new lengths,
//    advances the positions and clears the counters.
//
// Cross-workgroup data go through relaxed agent-scope atomics (coherent
// across the XCDs without cache-wide write-back or invalidation); the
// counters live in the workspace control block and return to zero.

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

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr int kDecThreads = 256;
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
__device__ __forceinline__ void row_store(const Row8<BF16>& r, void* base, int64_t elem) {
  if constexpr (BF16) {
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + elem) = r.w[0];
  } else {
    u32x4* p = reinterpret_cast<u32x4*>(reinterpret_cast<float*>(base) + elem);
    p[0] = r.w[0];
    p[1] = r.w[1];
  }
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

template <int D>
struct DecodeShape {
  static constexpr int LPE = D / 8;       // lanes per entry
  static constexpr int NGW = 64 / LPE;    // entry groups per wave
  static constexpr int NB = 4;            // entries per group
  static constexpr int TW = NGW * NB;     // entries per wave
  static constexpr int NWAVE = kDecThreads / 64;
  static constexpr int TWG = TW * NWAVE;  // entries per tile
  static constexpr int NP = NGW * NWAVE;  // partials per tile
};

__device__ __forceinline__ int tiles_of(int n, int twg) { return n <= 0 ? 1 : ceil_div(n, twg); }

// ---------------------------------------------------------------------------
// per-token work of one sequence, one of NS splits
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__device__ void token_work(const LayerArgs& a, const DecodeWs& w, int b, int sp) {
  constexpr int CW = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int HALF = D / 2;
  constexpr int HP = kDecThreads / D;  // query heads per split
  __shared__ float s_red[kDecThreads][8];
  __shared__ float s_cos[HALF], s_sin[HALF];
  __shared__ float s_q[HP * D];
  __shared__ float s_kt[HP][D];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int Hq = a.H_q, Hkv = a.H_kv, G = Hq / Hkv;
  const int Dm = a.D_model;
  const int C3 = 3 * Hkv, C = C3 + a.r;
  const int NS = w.splits;
  const int pos = a.next_pos[b];

  // ---- issue the loads of the rotation part first: q element and partner, key elements
  const int a0 = sp * HP, a1 = min(Hq, a0 + HP);
  const int qa = a0 + tid / D, qi = tid % D;
  const int64_t qbase = ((int64_t)b * Hq + min(qa, Hq - 1)) * D;
  const float qx = load_elem<BF16>(a.q, qbase + qi);
  const float qp = load_elem<BF16>(a.q, qbase + (qi < HALF ? qi + HALF : qi - HALF));
  const int h0 = a0 / G, h1 = (a1 - 1) / G;
  const int64_t kbase = ((int64_t)b * Hkv + min(h0 + wv, Hkv - 1)) * D;
  const float kx0 = load_elem<BF16>(a.k, kbase + (lane % HALF));
  const float kx1 = load_elem<BF16>(a.k, kbase + (lane % HALF) + HALF);

  // ---- partial gate projections over this split's rows of x [W_dec | W_dn].
  // Thread = (column group, row subset): a 16-byte chunk of CW columns when the
  // rows allow it, else a single column.
  const int RS = ceil_div(Dm, NS);
  const int r0 = sp * RS, r1 = min(Dm, r0 + RS);
  const bool vec = (C3 % CW == 0) && (a.r % CW == 0);
  const int nzc = vec ? C3 / CW : 0;
  const int nch = vec ? nzc + a.r / CW : C;  // column groups
  const int rstep = kDecThreads / nch;
  const int kc = tid % nch, rsub = tid / nch;
  const bool own = rsub < rstep;
  const bool dec_part = kc < (vec ? nzc : C3);
  const int mcols = dec_part ? C3 : a.r;
  const int mc0 = vec ? (dec_part ? kc : kc - nzc) * CW : (dec_part ? kc : kc - C3);
  const void* mbase = dec_part ? a.W_dec : a.W_dn;
  const int64_t xb = (int64_t)b * Dm;
  float acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.0f;
  constexpr int KR = 8;  // rows per thread per pass, all loads in flight together
  for (int rb = r0 + rsub; rb < r1; rb += KR * rstep) {
    float xr[KR];
    u32x4 raw[KR];
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const int row = min(rb + q * rstep, r1 - 1);
      xr[q] = load_elem<BF16>(a.x, xb + row);
      if (vec) {
        raw[q] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(mbase) +
                                                  ((int64_t)row * mcols + mc0) * (BF16 ? 2 : 4));
      } else {
        const float e = load_elem<BF16>(mbase, (int64_t)row * mcols + mc0);
        raw[q] = u32x4{__float_as_uint(e), 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const float xv = (own && rb + q * rstep < r1) ? xr[q] : 0.0f;
      if (vec) {
#pragma unroll
        for (int t = 0; t < CW; ++t) acc[t] = fmaf(xv, chunk_elem<BF16>(raw[q], t), acc[t]);
      } else {
        acc[0] = fmaf(xv, __uint_as_float(raw[q][0]), acc[0]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) s_red[tid][t] = acc[t];

  // ---- RoPE table (fp64 angles) while the loads fly
  if (tid < HALF) {
    double sn, cs;
    sincos((double)pos * a.inv_freq[tid], &sn, &cs);
    s_cos[tid] = (float)cs;
    s_sin[tid] = (float)sn;
  }
  __syncthreads();

  // ---- column sums of the partial projections -> workspace
  if (tid < C) {
    const int grp = vec ? (tid < C3 ? tid / CW : nzc + (tid - C3) / CW) : tid;
    const int t = vec ? (tid < C3 ? tid % CW : (tid - C3) % CW) : 0;
    float sum = 0.0f;
    for (int q = 0; q < rstep; ++q) sum += s_red[q * nch + grp][t];
    st_coh(w.zpart + ((int64_t)b * NS + sp) * w.zstride + tid, sum);
  }

  // ---- rotated queries of this split's heads
  if (qa < a1) {
    const float out =
        (qi < HALF) ? fmaf(qx, s_cos[qi], -qp * s_sin[qi]) : fmaf(qx, s_cos[qi - HALF], qp * s_sin[qi - HALF]);
    s_q[tid] = out;
    st_coh(w.qt + ((int64_t)b * Hq + qa) * D + qi, out);
  }
  // ---- the new key of each KV head the split touches (one wave each)
  if (wv <= h1 - h0) {
    const int h = h0 + wv;
    float k0 = (lane < HALF) ? kx0 : 0.0f;
    float k1 = (lane < HALF) ? kx1 : 0.0f;
    const float inv = 1.0f / fmaxf(sqrtf(wave_sum(k0 * k0 + k1 * k1)), 1e-12f);
    k0 *= inv;
    k1 *= inv;
    if (lane < HALF) {
      float rr0 = fmaf(k0, s_cos[lane], -k1 * s_sin[lane]);
      float rr1 = fmaf(k1, s_cos[lane], k0 * s_sin[lane]);
      if constexpr (BF16) {
        rr0 = bf16_to_f32(f32_to_bf16(rr0));
        rr1 = bf16_to_f32(f32_to_bf16(rr1));
      }
      s_kt[wv][lane] = rr0;
      s_kt[wv][lane + HALF] = rr1;
      if (h * G >= a0) {  // the split holding query head h G stores KV head h's key
        const int64_t kb = ((int64_t)b * Hkv + h) * D;
        st_coh(w.kt + kb + lane, rr0);
        st_coh(w.kt + kb + lane + HALF, rr1);
      }
    }
  }
  __syncthreads();
  // ---- the token's own logits (log2 units), one wave per query head
  if (a0 + wv < a1) {
    const int hw = (a0 + wv) / G - h0;
    float e = 0.0f;
    for (int i = lane; i < D; i += 64) e = fmaf(s_q[wv * D + i], s_kt[hw][i], e);
    e = wave_sum(e);
    if (lane == 0) st_coh(w.eself + b * Hq + a0 + wv, e * a.scale * kLog2e);
  }
  // ---- publish
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) add_coh(&w.tok_done[b], 1);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int D, int G, bool BF16, bool COMPACT>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(LayerArgs a, DecodeWs w, Control ctl, float tau,
                                                                  int32_t* kept) {
  using Sh = DecodeShape<D>;
  constexpr int LPE = Sh::LPE, NGW = Sh::NGW, NB = Sh::NB, TW = Sh::TW, TWG = Sh::TWG, NP = Sh::NP;
  constexpr int NT = kDecThreads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int S = a.B * a.H_kv;
  const int Hkv = a.H_kv;
  const int NS = w.splits;
  const int ntok = a.B * NS;

  __shared__ int s_id;
  __shared__ int s_scan[NT / 64 + 1];
  __shared__ int s_info[4];
  __shared__ int s_flag;
  __shared__ float s_po[NP * G * D];
  __shared__ float s_pm[NP * G];
  __shared__ float s_pl[NP * G];
  __shared__ float s_tq[(G + 1) * D];  // the token's rotated queries of the group, then its key
  __shared__ float s_g[2];             // query and similarity gates (log sigmoid)
  __shared__ float s_u[kMaxRank + 1];  // x W_dn, then the new key's gate
  __shared__ int s_cnt[NT / 64];
  __shared__ int s_pre;

  if (tid == 0) s_id = add_coh(&ctl.cmp_glob[0], 1);
  __syncthreads();
  const int id = s_id;

  if (id < ntok) {
    token_work<D, BF16>(a, w, id / NS, id - (id / NS) * NS);
  } else {
    // ---- (segment, tile) from the segment lengths (constant in this kernel)
    const int tix = id - ntok;
    bool have;
    {
      const int per = (S + NT - 1) / NT;
      const int sb = tid * per;
      const int se = min(S, sb + per);
      int mine = 0;
      for (int s = sb; s < se; ++s) mine += tiles_of(a.seg_len[s], TWG);
      int total;
      const int excl = block_exclusive_scan<NT>(mine, s_scan, &total);
      have = tix < total;
      if (have) {
        int run = excl;
        for (int s = sb; s < se; ++s) {
          const int nt = tiles_of(a.seg_len[s], TWG);
          if (tix >= run && tix < run + nt) {
            s_info[0] = s;
            s_info[1] = tix - run;
            s_info[2] = nt;
            s_info[3] = run;
          }
          run += nt;
        }
      }
      __syncthreads();
    }
    if (have) {
      const int seg = s_info[0];
      const int kt_ = s_info[1];
      const int ntile = s_info[2];  // tiles of this segment (all arrive)
      const int pbase = s_info[3];  // global index of its first tile
      const int b = seg / Hkv;
      const int h = seg - b * Hkv;
      const int len = a.seg_len[seg];
      const int cap = a.seg_cap[seg];
      const int64_t off = a.seg_off[seg];
      const float qs2 = a.scale * kLog2e;
      const int grp = lane / LPE;
      const int c = lane - grp * LPE;
      const int e0 = kt_ * TWG + wv * TW + grp * NB;

      // ---- cached entries: issue every load (from a clamped slot) before waiting for the token
      Row8<BF16> kr[NB], vr[NB];
      float lamv[NB], lkv[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const int64_t j = min(off + min(e0 + bb, max(len - 1, 0)), a.total_slots - 1);
        row_load<BF16>(kr[bb], a.K, j * D + 8 * c);
        row_load<BF16>(vr[bb], a.V, j * D + 8 * c);
        lamv[bb] = a.lam[j];
        lkv[bb] = a.lk[j];
      }

      // ---- wait for the sequence's token data, then stage it in LDS
      if (tid == 0) {
        int spins = 0;
        while (ldi_coh(&w.tok_done[b]) < NS) {
          if (++spins > kSpinLimitDec) {
            atomicOr(a.status, 2);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __syncthreads();
      for (int q = tid; q < (G + 1) * D; q += NT) {
        const int g = q / D, i = q - g * D;
        s_tq[q] = (g < G) ? ld_coh(w.qt + ((int64_t)b * a.H_q + h * G + g) * D + i)
                          : ld_coh(w.kt + (int64_t)seg * D + i);
      }
      if (tid < 2) {
        const int col = tid == 0 ? h : 2 * Hkv + h;  // query and similarity gates
        float z = a.b_dec[col];
        for (int sp = 0; sp < NS; ++sp) z += ld_coh(w.zpart + ((int64_t)b * NS + sp) * w.zstride + col);
        s_g[tid] = log_sigmoid(z);
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

      if constexpr (COMPACT) {
        // ---- live count of the tile.  Entries in tile order are (wave, group,
        // entry); lane grp * LPE + bb owns entry bb of its group.
        bool mine_live = false;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) mine_live = (c == bb) ? live[bb] : mine_live;
        const uint64_t mask = __ballot(c < NB && mine_live);
        if (lane == 0) s_cnt[wv] = __popcll(mask);
        // this tile's rows are all in registers now (the dot products used them)
        __syncthreads();
        int count = 0, wbase = 0;
#pragma unroll
        for (int w2 = 0; w2 < NT / 64; ++w2) {
          wbase += (w2 < wv) ? s_cnt[w2] : 0;
          count += s_cnt[w2];
        }
        // ---- look back over the earlier tiles of the segment for the destination
        if (wv == 0) {
          int* st = ctl.cmp_state + pbase;
          if (kt_ == 0) {
            if (lane == 0) {
              sti_coh(&st[0], (count << 2) | 2);
              s_pre = 0;
            }
          } else {
            if (lane == 0) sti_coh(&st[kt_], (count << 2) | 1);
            int prefix = 0;
            int cpos = kt_ - 1;  // next predecessor to examine
            int spins = 0;
            while (true) {
              const int pc2 = cpos - lane;  // lane l reads predecessor cpos - l
              const int sv = (pc2 >= 0) ? ldi_coh(&st[pc2]) : 2;
              const int flag = (pc2 >= 0) ? (sv & 3) : 2;  // tile -1 acts as prefix 0
              const int val = (pc2 >= 0) ? (sv >> 2) : 0;
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
              sti_coh(&st[kt_], ((prefix + count) << 2) | 2);
              s_pre = prefix;
            }
          }
          // No wait for the earlier tiles' loads is needed: a tile publishes
          // its count only after the barrier that follows the use of all its
          // rows, and the prefix above needed the count (or a later inclusive
          // value) of every earlier tile.
        }
        __syncthreads();
        // ---- stores of the survivors, in order
        const int P = s_pre;
        const int myrank =
            wbase + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const int rk = __shfl(myrank, grp * LPE + bb, 64);
          if (live[bb]) {
            const int64_t dst = off + P + rk;
            row_store<BF16>(kr[bb], a.K, dst * D + 8 * c);
            row_store<BF16>(vr[bb], a.V, dst * D + 8 * c);
            if (c == bb) {
              a.lam[dst] = newlam[bb];
              a.lk[dst] = lkv[bb];
              if (kept) kept[dst] = e0 + bb;
            }
          }
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
          if (ch) a.lam[off + e0 + c] = val;
        }
        __syncthreads();
      }

      // ---- merge the tile's partials -> workspace row pbase + kt_
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

      // ---- arrival; the last tile of the segment combines
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) s_flag = (add_coh(&w.cnt[seg], 1) == ntile - 1);
      __syncthreads();
      if (s_flag) {
        // output-gate weights of this thread's outputs, issued first
        constexpr int OPT = (G * D + NT - 1) / NT;
        constexpr int kUp = 16;
        const int Hq = a.H_q;
        const int r = a.r;
        float up[OPT][kUp];
#pragma unroll
        for (int u = 0; u < OPT; ++u) {
          const int idx = min(u * NT + tid, G * D - 1);
          const int col = (h * G) * D + idx;
#pragma unroll
          for (int q = 0; q < kUp; ++q) up[u][q] = load_elem<BF16>(a.W_up, (int64_t)min(q, r - 1) * Hq * D + col);
        }
        // u = x W_dn and the new key's gate, from the partial projections
        for (int q = tid; q <= r; q += NT) {
          const int col = q < r ? 3 * Hkv + q : Hkv + h;
          float z = q < r ? 0.0f : a.b_dec[Hkv + h];
          for (int sp = 0; sp < NS; ++sp) z += ld_coh(w.zpart + ((int64_t)b * NS + sp) * w.zstride + col);
          s_u[q] = q < r ? z : log_sigmoid(z);
        }
        // running merge per output (g, i): the new token's own term first
        float Mr[OPT], Lr[OPT], Or[OPT];
#pragma unroll
        for (int u = 0; u < OPT; ++u) {
          const int idx = u * NT + tid;
          if (idx < G * D) {
            const int g = idx / D;
            const int i = idx - g * D;
            Mr[u] = ld_coh(w.eself + b * Hq + h * G + g);
            Lr[u] = 1.0f;
            Or[u] = load_elem<BF16>(a.v, (int64_t)seg * D + i);
          }
        }
        constexpr int TC = 32;        // tiles per pass
        float* s_cm = s_po;           // [G][TC] tile maxima
        float* s_cl = s_po + G * TC;  // [G][TC] tile sums
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
        // ---- output gate and y (s_u was written before the barriers above)
#pragma unroll
        for (int u = 0; u < OPT; ++u) {
          const int idx = u * NT + tid;
          if (idx < G * D) {
            const int col = (h * G) * D + idx;
            float z = a.b_up ? a.b_up[col] : 0.0f;
#pragma unroll
            for (int q = 0; q < kUp; ++q)
              if (q < r) z = fmaf(s_u[q], up[u][q], z);
            for (int q = kUp; q < r; ++q) z = fmaf(s_u[q], load_elem<BF16>(a.W_up, (int64_t)q * Hq * D + col), z);
            const int64_t yo = (int64_t)b * Hq * D + col;
            const float yv = sigmoid(z) * (Or[u] / Lr[u]);
            if (a.y_bf16) {
              reinterpret_cast<uint16_t*>(a.y)[yo] = f32_to_bf16(yv);
            } else {
              reinterpret_cast<float*>(a.y)[yo] = yv;
            }
          }
        }
        // ---- the new entry: after the survivors when compacting.  The final
        // length is read once: the flags it comes from are cleared below.
        int pos = len;
        if constexpr (COMPACT) {
          if (tid == 0) s_pre = ldi_coh(&ctl.cmp_state[pbase + ntile - 1]) >> 2;
          __syncthreads();
          pos = s_pre;
        }
        const bool room = len < cap;
        if (room) {
          for (int i = tid; i < D; i += NT) {
            const float kv = s_tq[G * D + i];  // the key this tile staged
            const int64_t dst = (off + pos) * D + i;
            if constexpr (BF16) {
              reinterpret_cast<uint16_t*>(a.K)[dst] = f32_to_bf16(kv);  // exact: kv is bf16-rounded
              reinterpret_cast<uint16_t*>(a.V)[dst] = reinterpret_cast<const uint16_t*>(a.v)[(int64_t)seg * D + i];
            } else {
              reinterpret_cast<float*>(a.K)[dst] = kv;
              reinterpret_cast<float*>(a.V)[dst] = reinterpret_cast<const float*>(a.v)[(int64_t)seg * D + i];
            }
          }
        }
        if (tid == 0) {
          if (room) {
            a.lam[off + pos] = 0.0f;
            a.lk[off + pos] = s_u[r];
            if (COMPACT && kept) kept[off + pos] = len;
          } else {
            atomicOr(a.status, 1);
          }
          sti_coh(&w.newlen[seg], room ? pos + 1 : pos);
          sti_coh(&w.cnt[seg], 0);
        }
        if constexpr (COMPACT) {
          for (int t = tid; t < ntile; t += NT) sti_coh(&ctl.cmp_state[pbase + t], 0);
        }
      }
    }
  }

  // ---- the last workgroup overall commits lengths and positions, clears counters
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_flag = (add_coh(&ctl.cmp_glob[1], 1) == (int)gridDim.x - 1);
  __syncthreads();
  if (s_flag) {
    for (int s = tid; s < S; s += NT) a.seg_len[s] = ldi_coh(&w.newlen[s]);
    for (int b = tid; b < a.B; b += NT) {
      a.next_pos[b] += 1;
      sti_coh(&w.tok_done[b], 0);
    }
    if (tid == 0) {
      sti_coh(&ctl.cmp_glob[0], 0);
      sti_coh(&ctl.cmp_glob[1], 0);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int decode_tile_entries(int d) { return d == 64 ? DecodeShape<64>::TWG : DecodeShape<128>::TWG; }

static int decode_token_splits(const LayerArgs& a) { return (a.H_q * a.d + kDecThreads - 1) / kDecThreads; }

static int64_t decode_max_tiles(const LayerArgs& a, int twg) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  return a.total_slots / twg + S + 1;
}

// Scratch after the control block.
static size_t decode_layout(const LayerArgs& a, int twg, DecodeWs* w, char* base) {
  const int64_t S = (int64_t)a.B * a.H_kv;
  const int G = a.H_q / a.H_kv;
  const int64_t mt = decode_max_tiles(a, twg);
  const int NS = decode_token_splits(a);
  const int zs = (3 * a.H_kv + a.r + 3) / 4 * 4;
  size_t n = 0;
  auto take = [&](size_t bytes) {
    char* q = base ? base + n : nullptr;
    n += align_up(bytes, 256);
    return q;
  };
  float* qt = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q * a.d));
  float* kt = reinterpret_cast<float*>(take(sizeof(float) * S * a.d));
  float* zpart = reinterpret_cast<float*>(take(sizeof(float) * a.B * NS * zs));
  int* newlen = reinterpret_cast<int*>(take(sizeof(int) * S));
  float* eself = reinterpret_cast<float*>(take(sizeof(float) * a.B * a.H_q));
  float* part_o = reinterpret_cast<float*>(take(sizeof(float) * mt * G * a.d));
  float* part_ml = reinterpret_cast<float*>(take(sizeof(float) * mt * G * 2));
  if (w) {
    w->qt = qt;
    w->kt = kt;
    w->zpart = zpart;
    w->newlen = newlen;
    w->eself = eself;
    w->part_o = part_o;
    w->part_ml = part_ml;
    w->max_tiles = (int)mt;
    w->splits = NS;
    w->zstride = zs;
  }
  return n;
}

size_t decode_ws_bytes(const LayerArgs& a, int twg) { return decode_layout(a, twg, nullptr, nullptr); }

DecodeWs decode_ws_carve(const LayerArgs& a, const Control& ctl, void* scratch, int twg) {
  DecodeWs w{};
  decode_layout(a, twg, &w, reinterpret_cast<char*>(scratch));
  w.cnt = ctl.dec_cnt;
  w.tok_done = ctl.dec_cntb;
  return w;
}

template <int D, int G, bool BF16>
static hipError_t launch_step(const LayerArgs& a, const DecodeWs& w, const Control& ctl, float tau, bool compact,
                              int32_t* kept, hipStream_t st) {
  const int grid = a.B * w.splits + w.max_tiles;
  if (compact) {
    hipLaunchKernelGGL((decode_step_kernel<D, G, BF16, true>), dim3(grid), dim3(kDecThreads), 0, st, a, w, ctl, tau,
                       kept);
  } else {
    hipLaunchKernelGGL((decode_step_kernel<D, G, BF16, false>), dim3(grid), dim3(kDecThreads), 0, st, a, w, ctl, tau,
                       kept);
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
