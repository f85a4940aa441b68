// Stable in-place compaction of the pruned cache (gfx950).
//
// An entry whose log-bias fell below log p is evicted and never returns
// (paperlayer.ai summary, section 4.2; ai4snews page after Figure 1).  Each
// segment (one sequence, one KV head) is cut into chunks of CH entries and
// every chunk gets its own workgroup, so long segments spread over many CUs:
//
//  compact_count -- per chunk: number of live entries (logbias >= log p);
//                   also clears the per-call flags and the ticket counter.
//  compact_move  -- workgroups take chunk ids from an atomic ticket, so a
//                   chunk's predecessors in its segment are always running or
//                   done.  A chunk's destination is the sum of its
//                   predecessors' live counts.  It loads its live rows into
//                   registers, publishes "loaded", waits until every earlier
//                   chunk whose source range its destination overlaps has
//                   loaded too, then stores.  Destinations never exceed
//                   sources, so these waits are the only hazard.  Chunks with
//                   no dead entry at or before them move nothing.
//
// Live flags come from a wave ballot; ranks inside a wave from mbcnt; the
// block prefix from an LDS scan.

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

constexpr int kCompactThreads = 256;

template <int RB>  // row bytes of K / V
struct CompactShape {
  static constexpr int CH = RB <= 128 ? 256 : (RB <= 256 ? 128 : 64);  // entries per chunk
  static constexpr int P16 = RB / 16;                                  // 16-byte pieces per row
  static constexpr int PPT = CH * P16 / kCompactThreads;               // pieces per thread
};

struct CompactWs {
  int* live;      // [max_chunks] live entries per chunk
  int* loaded;    // [max_chunks] 1 once the chunk's rows are in registers
  int* done;      // [S] finished chunks per segment
  int* ticket;    // [1]
  int max_chunks;
};

static int compact_max_chunks(const LayerArgs& a, int ch) {
  return (int)(a.total_slots / ch + (int64_t)a.B * a.H_kv + 1);
}

static int compact_ch(const LayerArgs& a) {
  const int rb = a.d * (a.bf16 ? 2 : 4);
  return rb <= 128 ? 256 : (rb <= 256 ? 128 : 64);
}

size_t compact_ws_bytes(const LayerArgs& a) {
  const int mc = compact_max_chunks(a, compact_ch(a));
  const int64_t S = (int64_t)a.B * a.H_kv;
  return align_up(sizeof(int) * mc, 256) * 2 + align_up(sizeof(int) * S, 256) + 256;
}

static CompactWs compact_carve(const LayerArgs& a, void* ws) {
  const int mc = compact_max_chunks(a, compact_ch(a));
  const int64_t S = (int64_t)a.B * a.H_kv;
  char* p = reinterpret_cast<char*>(ws);
  CompactWs w;
  w.live = reinterpret_cast<int*>(p);
  p += align_up(sizeof(int) * mc, 256);
  w.loaded = reinterpret_cast<int*>(p);
  p += align_up(sizeof(int) * mc, 256);
  w.done = reinterpret_cast<int*>(p);
  p += align_up(sizeof(int) * S, 256);
  w.ticket = reinterpret_cast<int*>(p);
  w.max_chunks = mc;
  return w;
}

// Map a flat chunk id to (segment, chunk in segment) from the static
// capacities: chunks of segment s are ids [first_s, first_s + ceil(cap_s/CH)).
// Returns false if id is past the last chunk.  Block-wide (barriers inside).
struct ChunkPos {
  int seg, c, first, nch;
};

__device__ bool map_chunk(const int32_t* seg_cap, int S, int ch, int id, ChunkPos* out, int* s_scan, int* s_info) {
  const int per = (S + kCompactThreads - 1) / kCompactThreads;
  const int sb = threadIdx.x * per;
  const int se = min(S, sb + per);
  int mine = 0;
  for (int s = sb; s < se; ++s) mine += max(1, (seg_cap[s] + ch - 1) / ch);
  int total;
  const int excl = block_exclusive_scan<kCompactThreads>(mine, s_scan, &total);
  if (id >= total) return false;
  int run = excl;
  for (int s = sb; s < se; ++s) {
    const int n = max(1, (seg_cap[s] + ch - 1) / ch);
    if (id >= run && id < run + n) {
      s_info[0] = s;
      s_info[1] = id - run;
      s_info[2] = run;
      s_info[3] = n;
    }
    run += n;
  }
  __syncthreads();
  out->seg = s_info[0];
  out->c = s_info[1];
  out->first = s_info[2];
  out->nch = s_info[3];
  return true;
}

template <int CH>
__global__ __launch_bounds__(kCompactThreads) void compact_count(LayerArgs a, CompactWs w, float tau) {
  __shared__ int s_scan[kCompactThreads / 64 + 1];
  __shared__ int s_info[4];
  __shared__ int s_cnt[kCompactThreads / 64];
  const int S = a.B * a.H_kv;
  if (blockIdx.x == 0 && threadIdx.x == 0) *w.ticket = 0;
  if (blockIdx.x < S && threadIdx.x == 0) w.done[blockIdx.x] = 0;
  ChunkPos cp;
  if (!map_chunk(a.seg_cap, S, CH, blockIdx.x, &cp, s_scan, s_info)) return;
  const int len = a.seg_len[cp.seg];
  const int64_t off = a.seg_off[cp.seg];
  const int j0 = cp.c * CH;
  int n = 0;
  for (int t = threadIdx.x; t < CH; t += kCompactThreads) {
    const int j = j0 + t;
    if (j < len && a.lam[off + j] >= tau) ++n;
  }
  n = wave_isum(n);
  if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int i = 0; i < kCompactThreads / 64; ++i) tot += s_cnt[i];
    w.live[blockIdx.x] = tot;
    w.loaded[blockIdx.x] = 0;
  }
}

__device__ __forceinline__ int ld_acquire(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

template <int RB>
__global__ __launch_bounds__(kCompactThreads) void compact_move(LayerArgs a, CompactWs w, float tau, int32_t* kept) {
  using Sh = CompactShape<RB>;
  constexpr int CH = Sh::CH, P16 = Sh::P16, PPT = Sh::PPT;
  __shared__ int s_scan[kCompactThreads / 64 + 1];
  __shared__ int s_info[4];
  __shared__ int s_ticket;
  __shared__ int s_src[CH];
  __shared__ int s_prefix;
  __shared__ int s_last;
  const int S = a.B * a.H_kv;
  const int tid = threadIdx.x;

  if (tid == 0) s_ticket = atomicAdd(w.ticket, 1);
  __syncthreads();
  const int id = s_ticket;
  ChunkPos cp;
  if (!map_chunk(a.seg_cap, S, CH, id, &cp, s_scan, s_info)) return;
  const int seg = cp.seg;
  const int len = a.seg_len[seg];
  const int64_t off = a.seg_off[seg];
  const int j0 = cp.c * CH;
  const int nlive = w.live[id];

  // destination of this chunk = live entries in earlier chunks of the segment
  if (tid == 0) {
    int p = 0;
    for (int c2 = 0; c2 < cp.c; ++c2) p += w.live[cp.first + c2];
    s_prefix = p;
  }
  __syncthreads();
  const int P = s_prefix;
  const bool moves = (P != j0) || (nlive != min(CH, max(0, len - j0)));

  if (j0 < len && moves) {
    // compacted list of live source indices (stable)
    int nl_before = 0;
    for (int t0 = 0; t0 < CH; t0 += kCompactThreads) {
      const int j = j0 + t0 + tid;
      const bool lv = (t0 + tid < CH) && j < len && a.lam[off + j] >= tau;
      const uint64_t mask = __ballot(lv);
      const int lane = tid & 63;
      const int rank_w = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
      int tot;
      const int wbase = block_exclusive_scan<kCompactThreads>((lane == 0) ? __popcll(mask) : 0, s_scan, &tot);
      const int wave_off = __shfl(wbase, 0, 64);
      if (lv) s_src[nl_before + wave_off + rank_w] = t0 + tid;
      nl_before += tot;
      __syncthreads();
    }
    // load live rows (K, V pieces) and scalars into registers
    uint4 kreg[PPT], vreg[PPT];
    float lamr = 0.0f, lkr = 0.0f;
    int srcr = 0;
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int piece = u * kCompactThreads + tid;
      const int row = piece / P16;
      const int part = piece - row * P16;
      if (row < nlive) {
        const int64_t src = off + j0 + s_src[row];
        kreg[u] = reinterpret_cast<const uint4*>(a.K)[src * P16 + part];
        vreg[u] = reinterpret_cast<const uint4*>(a.V)[src * P16 + part];
      }
    }
    if (tid < nlive) {
      srcr = s_src[tid];
      lamr = a.lam[off + j0 + srcr];
      lkr = a.lk[off + j0 + srcr];
    }
    // every load has returned before the chunk is declared loaded
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&w.loaded[id], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);

    // wait for earlier chunks whose rows our destination overwrites
    if (tid == 0) {
      const int cfirst = P / CH;
      for (int c2 = cfirst; c2 < cp.c; ++c2) {
        int spins = 0;
        while (ld_acquire(&w.loaded[cp.first + c2]) == 0) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > (1 << 24)) {  // never expected; fail loudly, not forever
            atomicOr(a.status, 2);
            break;
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int piece = u * kCompactThreads + tid;
      const int row = piece / P16;
      const int part = piece - row * P16;
      if (row < nlive) {
        const int64_t dst = off + P + row;
        reinterpret_cast<uint4*>(a.K)[dst * P16 + part] = kreg[u];
        reinterpret_cast<uint4*>(a.V)[dst * P16 + part] = vreg[u];
      }
    }
    if (tid < nlive) {
      a.lam[off + P + tid] = lamr;
      a.lk[off + P + tid] = lkr;
      if (kept) kept[off + P + tid] = j0 + srcr;
    }
  } else {
    if (tid == 0) __hip_atomic_store(&w.loaded[id], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (kept && j0 < len) {
      for (int t = tid; t < nlive; t += kCompactThreads) kept[off + j0 + t] = j0 + t;
    }
  }

  // the last chunk of the segment sets the new length
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(&w.done[seg], 1);
    s_last = (old == cp.nch - 1);
  }
  __syncthreads();
  if (s_last && tid == 0) {
    __threadfence();
    int tot = 0;
    for (int c2 = 0; c2 < cp.nch; ++c2) tot += w.live[cp.first + c2];
    a.seg_len[seg] = tot;
  }
}

template <int RB>
static hipError_t launch_compact_rb(const LayerArgs& a, float tau, int32_t* kept, void* ws, hipStream_t st) {
  using Sh = CompactShape<RB>;
  CompactWs w = compact_carve(a, ws);
  hipLaunchKernelGGL((compact_count<Sh::CH>), dim3(w.max_chunks), dim3(kCompactThreads), 0, st, a, w, tau);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((compact_move<RB>), dim3(w.max_chunks), dim3(kCompactThreads), 0, st, a, w, tau, kept);
  return hipGetLastError();
}

hipError_t launch_compact(const LayerArgs& a, float tau, int32_t* kept, void* ws, hipStream_t st) {
  const int rb = a.d * (a.bf16 ? 2 : 4);
  switch (rb) {
    case 128: return launch_compact_rb<128>(a, tau, kept, ws, st);
    case 256: return launch_compact_rb<256>(a, tau, kept, ws, st);
    case 512: return launch_compact_rb<512>(a, tau, kept, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ua
