// Stable in-place compaction of the pruned cache (gfx950), one kernel.
//
// An entry whose log-bias fell below log p is evicted and never returns
// (paperlayer.ai summary, section 4.2; ai4snews page after Figure 1).  Each
// segment (one sequence, one KV head) is cut into chunks of CH entries, so
// long segments spread over many CUs.
//
// A persistent grid (at most one workgroup per CU) numbers the chunks of the
// segments' current lengths, segment by segment, and hands them out by an
// atomic ticket, so a chunk's predecessors in its segment were drawn earlier
// by running workgroups (every wait below is on a lower id, which guarantees
// progress).  Only chunks that hold entries are drawn: a grid sized by
// capacity would pay a ticket and an arrival per empty chunk, and those
// atomics on one word serialise.  Per chunk:
//  1. load the chunk's log-biases, count the live ones (ballot), publish the
//     count;
//  2. decoupled look-back over the predecessors' published counts/prefixes
//     (one wave reads up to 64 at once) gives the destination P of the
//     chunk's first survivor; publish the inclusive prefix;
//  3. if anything moves (P differs from the chunk start, or the chunk has a
//     hole): load the surviving rows into registers, publish "loaded", wait
//     until every earlier chunk whose rows the destination range overwrites
//     has loaded its own, then store.  Destinations never exceed sources, so
//     this is the only hazard.
// A workgroup draws tickets until one is past the last chunk, then reports
// done; the last one to report writes the new lengths (each segment's last
// inclusive prefix), clears the chunk flags and resets the counters.  The
// lengths stay unchanged until then, so every workgroup numbers the same
// chunks.  Flags use relaxed agent-scope atomics
// (coherent across XCDs without cache-wide maintenance); waits are bounded
// and report a timeout in status bit 1.

#include "ua_device.hpp"
#include "ua_kernels.hpp"

namespace ua {

// Two workgroup sizes: 256 threads for caches whose chunks are about as many
// as the grid's workgroups, 512 threads (chunks twice as long) for larger
// caches, where a workgroup walks several chunks in turn and fewer, longer
// chunks shorten that walk.
template <int RB, int NT>  // row bytes of K / V, threads per workgroup
struct CompactShape {
  static constexpr int CH = (RB <= 128 ? 256 : (RB <= 256 ? 128 : 64)) * NT / 256;  // entries per chunk
  static constexpr int P16 = RB / 16;                                                // 16-byte pieces per row
  static constexpr int PPT = CH * P16 / NT;                                          // pieces per thread
};

__device__ __forceinline__ int ldi_coh(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sti_coh2(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int addi_coh(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kSpinLimit = 1 << 22;
constexpr int kCompactGrid = 256;  // persistent workgroups (one per CU)

__device__ __forceinline__ int chunks_of(int len, int ch) { return len <= 0 ? 0 : (len + ch - 1) / ch; }

template <int RB, int kCompactThreads>
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(LayerArgs a, Control ctl, float tau, int32_t* kept) {
  using Sh = CompactShape<RB, kCompactThreads>;
  constexpr int CH = Sh::CH, P16 = Sh::P16, PPT = Sh::PPT;
  __shared__ int s_scan[kCompactThreads / 64 + 1];
  __shared__ int s_info[6];
  __shared__ int s_ticket;
  __shared__ int s_src[CH];
  __shared__ int s_cnt[kCompactThreads / 64];
  __shared__ int s_prefix;
  const int S = a.B * a.H_kv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;

  // ---- numbering from the lengths at the start of the call; a thread's
  // segments (up to MP of them) stay in registers, so finding a chunk's
  // segment later reads nothing
  constexpr int MP = 4;
  const int per = (S + kCompactThreads - 1) / kCompactThreads;
  const int sb = min(S, tid * per);
  const int se = min(S, sb + per);
  if (tid == 0) s_ticket = addi_coh(&ctl.glob[kGlobTicket], 1);
  int lenr[MP];
  int64_t offr[MP];
  int mine = 0;
  if (per <= MP) {
#pragma unroll
    for (int k = 0; k < MP; ++k) {
      lenr[k] = (sb + k < se) ? a.seg_len[sb + k] : 0;
      offr[k] = (sb + k < se) ? a.seg_off[sb + k] : 0;
    }
#pragma unroll
    for (int k = 0; k < MP; ++k) mine += chunks_of(lenr[k], CH);
  } else {
    for (int s = sb; s < se; ++s) mine += chunks_of(a.seg_len[s], CH);
  }
  int total;
  const int excl = block_exclusive_scan<kCompactThreads>(mine, s_scan, &total);

  bool first_draw = true;
  while (true) {
    // a ticket per chunk, drawn when the previous chunk is done (a ticket
    // drawn ahead would leave a low id waiting behind a busy workgroup, and
    // every later chunk's look-back on it)
    if (!first_draw && tid == 0) s_ticket = addi_coh(&ctl.glob[kGlobTicket], 1);
    first_draw = false;
    __syncthreads();
    const int id = s_ticket;

    if (id >= total || id < 0) {  // (a negative id only from a corrupted ticket word: touch no chunk)
      // ---- exit: report done; the last workgroup to report commits (every
      // other one has stored its rows and published its chunks by then)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) s_ticket = addi_coh(&ctl.glob[kGlobArrive], 1);
      __syncthreads();
      if (s_ticket == (int)gridDim.x - 1) {
        int run = excl;
        for (int s = sb; s < se; ++s) {
          const int n = chunks_of(a.seg_len[s], CH);
          if (n > 0) a.seg_len[s] = ldi_coh(&ctl.cmp_state[run + n - 1]) >> 2;
          run += n;
        }
        __syncthreads();  // every prefix read before any flag is cleared
        for (int t = tid; t < total; t += kCompactThreads) {
          sti_coh2(&ctl.cmp_state[t], 0);
          sti_coh2(&ctl.cmp_loaded[t], 0);
        }
        if (tid == 0) {
          sti_coh2(&ctl.glob[kGlobTicket], 0);
          sti_coh2(&ctl.glob[kGlobArrive], 0);
        }
      }
      break;
    }

    // ---- chunk id -> (segment, chunk, first chunk of the segment, length, offset)
    if (id >= excl && id < excl + mine) {
      int run = excl;
      if (per <= MP) {
#pragma unroll
        for (int k = 0; k < MP; ++k) {
          const int n = chunks_of(lenr[k], CH);
          if (id >= run && id < run + n) {
            s_info[0] = sb + k;
            s_info[1] = id - run;
            s_info[2] = run;
            s_info[3] = (int)(uint32_t)(offr[k] & 0xffffffff);
            s_info[4] = (int)(offr[k] >> 32);
            s_info[5] = lenr[k];
          }
          run += n;
        }
      } else {
        for (int s = sb; s < se; ++s) {
          const int n = chunks_of(a.seg_len[s], CH);
          if (id >= run && id < run + n) {
            const int64_t o = a.seg_off[s];
            s_info[5] = a.seg_len[s];
            s_info[0] = s;
            s_info[1] = id - run;
            s_info[2] = run;
            s_info[3] = (int)(uint32_t)(o & 0xffffffff);
            s_info[4] = (int)(o >> 32);
          }
          run += n;
        }
      }
    }
    __syncthreads();
    const int seg = s_info[0];
    const int c = s_info[1];
    const int first = s_info[2];
    const int len = s_info[5];
    const int64_t off = (int64_t)(uint32_t)s_info[3] | ((int64_t)s_info[4] << 32);
    const int j0 = c * CH;
    const int nvalid = min(CH, len - j0);  // >= 1: only chunks with entries are numbered

    // 1. live flags and count
    const int j = j0 + tid;
    float lamr = 0.0f;
    bool lv = false;
    if (tid < CH && j < len) {
      lamr = a.lam[off + j];
      lv = lamr >= tau;
    }
    const uint64_t mask = __ballot(lv);
    if (lane == 0) s_cnt[wv] = __popcll(mask);
    __syncthreads();
    int count = 0;
#pragma unroll
    for (int w2 = 0; w2 < kCompactThreads / 64; ++w2) count += s_cnt[w2];

    // 2. publish, then look back for the destination of the first survivor
    if (wv == 0) {
      if (c == 0) {
        if (lane == 0) {
          sti_coh2(&ctl.cmp_state[id], (count << 2) | 2);
          s_prefix = 0;
        }
      } else {
        if (lane == 0) sti_coh2(&ctl.cmp_state[id], (count << 2) | 1);
        int prefix = 0;
        int cpos = c - 1;  // next predecessor to examine
        int spins = 0;
        while (true) {
          const int pc = cpos - lane;  // lane l reads predecessor cpos - l
          int st = (pc >= 0) ? ldi_coh(&ctl.cmp_state[first + pc]) : 2;  // chunk -1 acts as prefix 0
          const int flag = (pc >= 0) ? (st & 3) : 2;
          const int val = (pc >= 0) ? (st >> 2) : 0;
          // first lane (nearest predecessor) whose prefix is complete
          const uint64_t inc = __ballot(flag == 2);
          const uint64_t none = __ballot(flag == 0);
          const int stop = inc ? (int)__builtin_ctzll(inc) : 64;
          // every lane up to `stop` must have published at least its count
          const uint64_t need = (stop >= 63) ? ~0ull : ((2ull << stop) - 1);
          if ((none & need) == 0) {
            int contrib = (lane <= stop) ? val : 0;
            contrib = wave_isum(contrib);
            prefix += contrib;
            if (stop < 64) break;
            cpos -= 64;
            continue;
          }
          if (++spins > kSpinLimit) {
            if (lane == 0) atomicOr(a.status, 2);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) {
          sti_coh2(&ctl.cmp_state[id], ((prefix + count) << 2) | 2);
          s_prefix = prefix;
        }
      }
    }
    __syncthreads();
    const int P = s_prefix;
    const bool moves = (P != j0) || (count != nvalid);

    if (moves) {
      // stable list of survivors (chunk-relative source indices)
      {
        const int rank_w = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
        int wbase = 0;
        for (int w2 = 0; w2 < wv; ++w2) wbase += s_cnt[w2];
        if (lv) s_src[wbase + rank_w] = tid;
      }
      __syncthreads();
      // unconditional loads from a clamped row (always inside this chunk) keep
      // the rows in registers; only the stores below are predicated
      u32x4 kreg[PPT], vreg[PPT];
      float lkr = 0.0f, lsv = 0.0f;
      int srcr = 0;
      const int64_t cbase = off + j0;
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int piece = u * kCompactThreads + tid;
        const int row = piece / P16;
        const int part = piece - row * P16;
        const int rsrc = (count > 0) ? s_src[row < count ? row : 0] : 0;
        const int64_t src = cbase + rsrc;
        kreg[u] = reinterpret_cast<const u32x4*>(a.K)[src * P16 + part];
        vreg[u] = reinterpret_cast<const u32x4*>(a.V)[src * P16 + part];
      }
      if (tid < count) {
        srcr = s_src[tid];
        lsv = a.lam[off + j0 + srcr];
        lkr = a.lk[off + j0 + srcr];
      }
      __builtin_amdgcn_s_waitcnt(0);  // every row is in registers
      __syncthreads();
      if (tid == 0) sti_coh2(&ctl.cmp_loaded[id], 1);
      // wait for the earlier chunks whose rows the destination overwrites
      if (wv == 0) {
        const int cfirst = P / CH;
        int spins = 0;
        for (int cb = cfirst; cb < c; cb += 64) {
          const int cc = cb + lane;
          while (true) {
            const int ok = (cc < c) ? ldi_coh(&ctl.cmp_loaded[first + cc]) : 1;
            if (__ballot(ok == 0) == 0) break;
            if (++spins > kSpinLimit) {
              if (lane == 0) atomicOr(a.status, 2);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int piece = u * kCompactThreads + tid;
        const int row = piece / P16;
        const int part = piece - row * P16;
        if (row < count) {
          const int64_t dst = off + P + row;
          reinterpret_cast<u32x4*>(a.K)[dst * P16 + part] = kreg[u];
          reinterpret_cast<u32x4*>(a.V)[dst * P16 + part] = vreg[u];
        }
      }
      if (tid < count) {
        a.lam[off + P + tid] = lsv;
        a.lk[off + P + tid] = lkr;
        if (kept) kept[off + P + tid] = j0 + srcr;
      }
    } else {
      if (tid == 0) sti_coh2(&ctl.cmp_loaded[id], 1);
      if (kept && tid < nvalid) kept[off + j0 + tid] = j0 + tid;
    }
    __syncthreads();  // shared state is rewritten by the next chunk
  }
}

template <int RB>
static hipError_t launch_rb(const LayerArgs& a, const Control& ctl, float tau, int32_t* kept, hipStream_t st) {
  const int grid = ctl.max_chunks < kCompactGrid ? ctl.max_chunks : kCompactGrid;
  // chunks of 256-thread workgroups the capacity allows, against the grid
  const int64_t cap_chunks = a.total_slots / CompactShape<RB, 256>::CH;
  if (cap_chunks > 2 * (int64_t)kCompactGrid) {
    hipLaunchKernelGGL((compact_kernel<RB, 512>), dim3(grid), dim3(512), 0, st, a, ctl, tau, kept);
  } else {
    hipLaunchKernelGGL((compact_kernel<RB, 256>), dim3(grid), dim3(256), 0, st, a, ctl, tau, kept);
  }
  return hipGetLastError();
}

hipError_t launch_compact(const LayerArgs& a, const Control& ctl, float tau, int32_t* kept, hipStream_t st) {
  const int rb = a.d * (a.bf16 ? 2 : 4);
  switch (rb) {
    case 128: return launch_rb<128>(a, ctl, tau, kept, st);
    case 256: return launch_rb<256>(a, ctl, tau, kept, st);
    case 512: return launch_rb<512>(a, ctl, tau, kept, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ua
