// Resolve one wave of a layer call against the global LRU pool of expert
// slots, and group the wave's (token, rank) pairs by expert.
//
// Pages: the GPU keeps a least-recently-used cache of expert slots shared by
// all layers; an expert already cached runs in place, a miss is streamed over
// PCIe; the hybrid strategy splits a step's misses between host compute and
// streaming (devpik article "FreeToken: Run Frontier MoE Models on Your Own
// GPU...", section "Why a Huge MoE Model Fits on One Consumer GPU"); prefill
// copies every expert of a layer per chunk (same article, "Long Prompts Are
// the Bottleneck").  Readings where the pages are silent (also stated in the
// oracle): a wave is the longest run of tokens whose union of experts fits the
// pool and is resolved as a set; victims are free slots by index, then the
// least recently used non-hit slots; one clock tick per pair.
//
// Device design: one 1024-thread workgroup.  The pool's recency order is kept
// as an array `lru` of all C slots (free slots first by index, then resident
// slots by last use), so victim selection is one prefix scan over `lru` that
// skips this wave's hit slots, and the update is a stable compaction of the
// untouched entries followed by the touched slots in order of their last pair.
// Pairs are grouped in first-appearance order (D order); each pair's rank in
// its group comes from a wavefront-ballot match of equal groups plus a
// per-wave prefix, so rows keep pair order inside a group without atomics.
#include "common.h"
#include "topk.h"

namespace ftmoe {

namespace {

constexpr int NT = kResolveThreads;
constexpr int NW = NT / 64;
constexpr int kLdsPairs = 2048;  // pairs of a wave kept in LDS (decode calls with T*k up to this)
constexpr int kPf = 4;           // recency-order entries per thread read at kernel start (C <= 4096)

// A descriptor's fields other than its tokens (which other threads write)
__device__ inline void put_desc_head(GroupDesc& d, uint64_t wptr, int row_begin, int row_count, int expert, int slot) {
  d.wptr = wptr;
  d.row_begin = row_begin;
  d.row_count = row_count;
  d.expert = expert;
  d.slot = slot;
}

struct ResolveSmem {
  int first[kMaxExperts];
  int last[kMaxExperts];
  int dix[kMaxExperts];
  int cnt[kMaxExperts];
  int D[kMaxExperts];
  int cls[kMaxExperts];
  int dslot[kMaxExperts];
  int mpos[kMaxExperts];
  int gpos[kMaxExperts];  // position of each group in the run list
  int tbase[kMaxExperts]; // prefill: each group's first row tile in the MX GEMM work list
  int off[kMaxExperts];
  int sm[kMaxExperts];
  int wcnt[NW][kMaxExperts];
  int wbuf[2][NW];
  int scal[16];
  uint32_t prot[kMaxSlots / 32];  // slots hit by this wave (not evictable)
  int ired[4 * NW];
  double dred[NW];
  int k2s[kMaxExperts];           // key -> slot of this layer's experts, read at start
  // the wave's pairs mirrored in LDS when P <= kLdsPairs (decode calls)
  int32_t psel[kLdsPairs];
  float pw[kLdsPairs];
  int32_t prow[kLdsPairs];
  double pgap[kLdsPairs];
  uint32_t lastbits[kLdsPairs / 32];  // positions of the touched experts' last pairs
  int lastpre[kLdsPairs / 32];
};

// ---- workgroup scans and reductions without LDS round trips inside a wave:
// DPP row operations plus readlanes across the four rows of 16 lanes.  The
// per-wave totals meet in LDS; two alternating buffers let a scan skip the
// barrier that would otherwise protect the buffer from the next scan.
template <int CTRL>
__device__ __attribute__((always_inline)) inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// inclusive prefix sum over the wavefront
__device__ __attribute__((always_inline)) inline int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
  x += dpp_i<0x111>(x);  // row_shr:1
  x += dpp_i<0x112>(x);  // row_shr:2
  x += dpp_i<0x114>(x);  // row_shr:4
  x += dpp_i<0x118>(x);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// every lane of a row of 16 gets the row's sum / max (butterfly inside the row)
__device__ __attribute__((always_inline)) inline int row_sum(int x) {
  x += dpp_i<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_i<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_i<0x141>(x);  // row_half_mirror
  x += dpp_i<0x140>(x);  // row_mirror
  return x;
}
__device__ __attribute__((always_inline)) inline int row_max(int x) {
  x = max(x, dpp_i<0xB1>(x));
  x = max(x, dpp_i<0x4E>(x));
  x = max(x, dpp_i<0x141>(x));
  x = max(x, dpp_i<0x140>(x));
  return x;
}
template <int CTRL>
__device__ __attribute__((always_inline)) inline double dpp_d(double v) {
  const uint64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(int(uint32_t(b)), int(uint32_t(b)), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(int(uint32_t(b >> 32)), int(uint32_t(b >> 32)), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((int64_t(uint32_t(hi)) << 32) | uint32_t(lo));
}
__device__ __attribute__((always_inline)) inline double row_min(double x) {
  x = fmin(x, dpp_d<0xB1>(x));
  x = fmin(x, dpp_d<0x4E>(x));
  x = fmin(x, dpp_d<0x141>(x));
  x = fmin(x, dpp_d<0x140>(x));
  return x;
}
__device__ __attribute__((always_inline)) inline int wave_sum(int x) {
  x = row_sum(x);
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) + __builtin_amdgcn_readlane(x, 32) +
         __builtin_amdgcn_readlane(x, 48);
}
__device__ __attribute__((always_inline)) inline int wave_max(int x) {
  x = row_max(x);
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __attribute__((always_inline)) inline double readlane_d(double v, int src) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(b), src);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(b >> 32), src);
  return __longlong_as_double((int64_t(hi) << 32) | lo);
}
__device__ __attribute__((always_inline)) inline double wave_min(double x) {
  x = row_min(x);
  return fmin(fmin(readlane_d(x, 0), readlane_d(x, 16)), fmin(readlane_d(x, 32), readlane_d(x, 48)));
}

// Wave totals of the block scans, in two alternating buffers.
// Exclusive prefix sum of v over the workgroup; *total gets the sum.  par
// (uniform, per thread) selects the buffer and flips.
__device__ __attribute__((always_inline)) inline int block_exscan(int v, int (&wbuf)[2][NW], int& par,
                                                                  int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wbuf[par][wid] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int s = wbuf[par][w];
    pre += (w < wid) ? s : 0;
    tot += s;
  }
  par ^= 1;
  *total = tot;
  return pre + incl - v;
}

// Exclusive count of set flags over the workgroup (ballot within the wave).
__device__ __attribute__((always_inline)) inline int block_excount(bool f, int (&wbuf)[2][NW], int& par,
                                                                   int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  const int below = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
  if (lane == 0) wbuf[par][wid] = __popcll(m);
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int s = wbuf[par][w];
    pre += (w < wid) ? s : 0;
    tot += s;
  }
  par ^= 1;
  *total = tot;
  return pre + below;
}

// One pass for the call's closing counters: three sums, a max and an fp64 min
// (one barrier; its buffers are used once per kernel).
struct Closing {
  int cpu_rows, hit_pairs, stream_rows, max_rows;
  double min_gap;
};

__device__ Closing block_closing(int cpu_rows, int hit_pairs, int stream_rows, int max_rows, double gap, int* ired,
                                 double* dred) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  cpu_rows = wave_sum(cpu_rows);
  hit_pairs = wave_sum(hit_pairs);
  stream_rows = wave_sum(stream_rows);
  max_rows = wave_max(max_rows);
  gap = wave_min(gap);
  if (lane == 0) {
    ired[4 * wid + 0] = cpu_rows;
    ired[4 * wid + 1] = hit_pairs;
    ired[4 * wid + 2] = stream_rows;
    ired[4 * wid + 3] = max_rows;
    dred[wid] = gap;
  }
  __syncthreads();
  Closing c{0, 0, 0, 0, __builtin_inf()};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    c.cpu_rows += ired[4 * w + 0];
    c.hit_pairs += ired[4 * w + 1];
    c.stream_rows += ired[4 * w + 2];
    c.max_rows = max(c.max_rows, ired[4 * w + 3]);
    c.min_gap = fmin(c.min_gap, dred[w]);
  }
  return c;
}

__global__ __launch_bounds__(NT) void k_resolve(ResolveArgs a) {
  __shared__ ResolveSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int E = a.E, k = a.k, C = a.C, t0 = a.t0;
  int par = 0;  // scan buffer parity
  const bool decode = a.mode == 0;
  const int key0 = a.layer * E;

  // ---- prologue: every global read that does not depend on this call's
  // routing is issued first, so that its latency overlaps the top-k: the
  // recency order and the keys held by its first slots, this layer's
  // key -> slot entries, the clock and the counters.
  int cur = 0;
  uint64_t clk = 0;
  int k2s = -1;
  const bool use_k2s = decode || a.stage_hits != 0;
  if (use_k2s) {
    cur = *a.tab.lru_cur;
    clk = *a.tab.clock;
  }
  if (use_k2s && tid < E) k2s = a.tab.key2slot[key0 + tid];
  uint64_t* st = a.tab.stats + int64_t(a.layer) * ST_COUNT;
  uint64_t st0[ST_COUNT];
  double gap0 = 0.0;
  uint64_t pc0[3][2] = {{0, 0}, {0, 0}, {0, 0}};
  if (tid == 0) {
#pragma unroll
    for (int i = 0; i < ST_COUNT; ++i) st0[i] = st[i];
    gap0 = a.tab.min_gap[a.layer];
    if (a.prof_cnt != nullptr)
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        pc0[i][0] = a.prof_cnt[(i * 4 + a.fmt) * 2];
        pc0[i][1] = a.prof_cnt[(i * 4 + a.fmt) * 2 + 1];
      }
  }
  const int32_t* lru_in = a.tab.lru[cur];
  // both recency buffers, so that these loads need not wait for lru_cur
  int pf_s[kPf], pf_key[kPf];
  {
    int pf0[kPf], pf1[kPf];
#pragma unroll
    for (int j = 0; j < kPf; ++j) {
      const int i = j * NT + tid;
      const bool ok = decode && i < C;
      pf0[j] = ok ? a.tab.lru[0][i] : 0;
      pf1[j] = ok ? a.tab.lru[1][i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kPf; ++j) pf_s[j] = cur ? pf1[j] : pf0[j];
  }

  // ---- 0. top-k of every token of the call (first wave of a decode call)
  const bool mirror = a.do_topk && int64_t(a.T) * k <= kLdsPairs;
  if (a.do_topk) {
    for (int t = wid; t < a.T; t += NW)
      wave_topk(a.z + int64_t(t) * E, E, k, a.sel + int64_t(t) * k, a.w + int64_t(t) * k, a.gap + t,
                mirror ? sm.psel + t * k : nullptr, mirror ? sm.pw + t * k : nullptr, mirror ? sm.pgap + t : nullptr);
    // later phases read the global copies only without the LDS mirror
    if (!mirror) __threadfence_block();
  }
  // keys of the prefetched recency entries (the old key of a victim slot)
#pragma unroll
  for (int j = 0; j < kPf; ++j) {
    const int i = j * NT + tid;
    pf_key[j] = (decode && i < C) ? a.tab.slot_key[pf_s[j]] : -1;
  }
  if (use_k2s && tid < E) sm.k2s[tid] = k2s;
  for (int e = tid; e < E; e += NT) {
    sm.first[e] = 0x7fffffff;
    sm.last[e] = -1;
    sm.dix[e] = 0;
    sm.cnt[e] = 0;
  }
  __syncthreads();

  // ---- 1. end of the wave: tokens while the union of experts fits C
  if (tid == 0) sm.scal[0] = a.T;
  if (decode && C < E && wid == 0) {
    int count = 0, t1 = a.T;
    for (int t = t0; t < a.T; ++t) {
      const int e = lane < k ? (mirror ? sm.psel[t * k + lane] : a.sel[int64_t(t) * k + lane]) : 0;
      const bool isnew = lane < k && sm.dix[e] == 0;
      const int n = __popcll(__ballot(isnew));
      if (count + n > C) {
        t1 = t;
        break;
      }
      if (isnew) sm.dix[e] = 1;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      count += n;
    }
    if (lane == 0) sm.scal[0] = t1 > t0 ? t1 : t0 + 1;
  }
  __syncthreads();
  const int t1 = sm.scal[0];
  const int P = (t1 - t0) * k;
  const int ntok = t1 - t0;
  const int64_t pb = int64_t(t0) * k;
  for (int e = tid; e < E; e += NT) sm.dix[e] = -1;

  // pairs of this wave in LDS: already there from the top-k, else one copy
  const bool lp = P <= kLdsPairs;
  if (lp && !mirror) {
    for (int i = tid; i < P; i += NT) {
      sm.psel[i] = a.sel[pb + i];
      sm.pw[i] = a.w[pb + i];
    }
    for (int tt = tid; tt < ntok; tt += NT) sm.pgap[tt] = a.gap[t0 + tt];
    __syncthreads();
  }
  auto SEL = [&](int i) -> int { return lp ? sm.psel[i] : a.sel[pb + i]; };

  int nD = 0;
  const bool agg = a.agg != nullptr;  // staged call spread over workgroups
  if (!agg) {
    // ---- 2. first and last pair of each expert in the wave
    for (int i = tid; i < P; i += NT) {
      const int e = SEL(i);
      atomicMin(&sm.first[e], i);
      atomicMax(&sm.last[e], i);
    }
    __syncthreads();

    // ---- 3. D: distinct experts in order of first appearance
    for (int c0 = 0; c0 < P; c0 += NT) {
      const int i = c0 + tid;
      int e = 0;
      bool f = false;
      if (i < P) {
        e = SEL(i);
        f = sm.first[e] == i;
      }
      int tot;
      const int pos = block_excount(f, sm.wbuf, par, &tot);
      if (f) {
        sm.D[nD + pos] = e;
        sm.dix[e] = nD + pos;
      }
      nD += tot;
    }
    __syncthreads();
  } else {
    // ---- 2-3 from the per-chunk histograms (k_stage_hist): each expert's
    // first and last pair and count, and the exclusive prefix of its count
    // over the chunks (the row base of its pairs in each chunk, for
    // k_stage_rows).  Thread (j, e) takes a contiguous run of chunks.
    const int nc = a.nchunks;
    const int32_t* hist = a.agg;
    const int32_t* cfirst = hist + int64_t(nc) * E;
    const int32_t* clast = cfirst + int64_t(nc) * E;
    int32_t* cbase = const_cast<int32_t*>(clast) + int64_t(nc) * E;
    const int J = max(1, NT / E);
    const int e = tid % E, j = tid / E;
    const int per = (nc + J - 1) / J;
    const int c_lo = min(nc, j * per), c_hi = min(nc, c_lo + per);
    int* tcnt = &sm.wcnt[0][0];  // [J][E] scratch (the rank tables are not used here)
    int* tfirst = tcnt + NT;
    int* tlast = tfirst + NT;
    const bool mine = tid < J * E;
    int n = 0, f = 0x7fffffff, l = -1;
    if (mine)
      for (int c = c_lo; c < c_hi; ++c) {
        n += hist[int64_t(c) * E + e];
        f = min(f, cfirst[int64_t(c) * E + e]);
        l = max(l, clast[int64_t(c) * E + e]);
      }
    if (mine) {
      tcnt[j * E + e] = n;
      tfirst[j * E + e] = f;
      tlast[j * E + e] = l;
    }
    __syncthreads();
    if (mine) {
      int run = 0;
      for (int j2 = 0; j2 < j; ++j2) run += tcnt[j2 * E + e];
      for (int c = c_lo; c < c_hi; ++c) {
        cbase[int64_t(c) * E + e] = run;
        run += hist[int64_t(c) * E + e];
      }
    }
    if (tid < E) {
      int tn = 0, tf = 0x7fffffff, tl = -1;
      for (int j2 = 0; j2 < J; ++j2) {
        tn += tcnt[j2 * E + tid];
        tf = min(tf, tfirst[j2 * E + tid]);
        tl = max(tl, tlast[j2 * E + tid]);
      }
      sm.first[tid] = tf;
      sm.last[tid] = tl;
      sm.off[tid] = tn;  // the expert's count until its D position is known
    }
    __syncthreads();
    // D order: rank of each selected expert by its first pair
    const bool sel_e = tid < E && sm.off[tid] > 0;
    int rank = 0;
    if (sel_e) {
      const int myf = sm.first[tid];
      for (int e2 = 0; e2 < E; ++e2) rank += (sm.off[e2] > 0 && sm.first[e2] < myf) ? 1 : 0;
    }
    (void)block_excount(sel_e, sm.wbuf, par, &nD);
    if (sel_e) {
      sm.D[rank] = tid;
      sm.dix[tid] = rank;
      sm.cnt[rank] = sm.off[tid];
    }
    __syncthreads();
  }

  // ---- 4. hits, misses, hybrid split
  if (decode) {
    for (int i = tid; i < (C + 31) / 32; i += NT) sm.prot[i] = 0u;
    __syncthreads();
  }
  int hit = 0;
  if (tid < nD) {
    const int e = sm.D[tid];
    if (decode) {
      const int s = sm.k2s[e];
      hit = s >= 0;
      if (hit) {
        sm.dslot[tid] = s;
        atomicOr(&sm.prot[s >> 5], 1u << (s & 31));
      }
    } else {
      // staged: a resident expert (outside the staging region, which was
      // cleared before this kernel) is read from its slot
      const int s = a.stage_hits ? sm.k2s[e] : -1;
      hit = s >= 0;
      sm.dslot[tid] = hit ? s : (a.layer & 1) * E + e;
    }
  }
  int nM;
  const int mp = block_excount(tid < nD && !hit, sm.wbuf, par, &nM);
  // IEEE double, no contraction: floor(nM * share + 1/2)
  const int m_cpu = decode ? int(floor(__dadd_rn(__dmul_rn(double(nM), a.share), 0.5))) : 0;
  const int m_str = nM - m_cpu;
  if (tid < nD) {
    sm.mpos[tid] = hit ? -1 : mp;
    const int c = hit ? FT_PAIR_HIT : (mp < m_str ? FT_PAIR_MISS_STREAM : FT_PAIR_MISS_CPU);
    sm.cls[tid] = c;
    if (c == FT_PAIR_MISS_STREAM) sm.sm[mp] = tid;
  }
  if (tid == 0) sm.scal[1] = 0;  // evictions
  __syncthreads();

  // ---- 5b. hit-D2D staging: the copied experts (not resident elsewhere)
  // become residents of their staging slots, and the call updates the
  // recency order like one wave over its pairs -- copies no token selects
  // first (one clock tick each, in expert order), then every selected expert
  // (read in place or copied) at the clock of its last pair.  The staging
  // halves were cleared before this kernel, so a copy's slot is free here.
  // New order: free slots ascending, residents this call does not touch in
  // their old order, unselected copies, selected experts by last pair.
  if (!decode && a.stage_hits) {
    const int base = (a.layer & 1) * E;
    for (int i = tid; i < (C + 31) / 32; i += NT) sm.prot[i] = 0u;
    __syncthreads();
    if (tid < nD && sm.cls[tid] == FT_PAIR_HIT) {
      const int s = sm.dslot[tid];
      atomicOr(&sm.prot[s >> 5], 1u << (s & 31));
    }
    const bool copied = tid < E && sm.k2s[tid] < 0;
    const bool unsel = copied && sm.last[tid] < 0;
    int u;
    const int ur = block_excount(unsel, sm.wbuf, par, &u);  // its barrier publishes the marks above
    int32_t* lru_out = a.tab.lru[cur ^ 1];
    int nfree = 0;
    for (int c0 = 0; c0 < C; c0 += NT) {
      const int s = c0 + tid;
      bool f = false;
      if (s < C) {
        const bool reg = s >= base && s < base + E && sm.k2s[s - base] < 0;
        f = !reg && a.tab.slot_key[s] < 0;
      }
      int tot;
      const int p = block_excount(f, sm.wbuf, par, &tot);
      if (f) lru_out[nfree + p] = s;
      nfree += tot;
    }
    int nold = 0;
    for (int c0 = 0; c0 < C; c0 += NT) {
      const int i = c0 + tid;
      int s = 0;
      bool r = false;
      if (i < C) {
        s = lru_in[i];
        r = a.tab.slot_key[s] >= 0 && !((sm.prot[s >> 5] >> (s & 31)) & 1u);
      }
      int tot;
      const int p = block_excount(r, sm.wbuf, par, &tot);
      if (r) lru_out[nfree + nold + p] = s;
      nold += tot;
    }
    if (unsel) {
      lru_out[nfree + nold + ur] = base + tid;
      a.tab.slot_last[base + tid] = clk + uint64_t(ur);
    }
    for (int d = tid; d < nD; d += NT) {
      const int mylast = sm.last[sm.D[d]];
      int rank = 0;
      for (int d2 = 0; d2 < nD; ++d2) rank += sm.last[sm.D[d2]] < mylast ? 1 : 0;
      lru_out[nfree + nold + u + rank] = sm.dslot[d];
      a.tab.slot_last[sm.dslot[d]] = clk + uint64_t(u) + uint64_t(mylast);
    }
    __syncthreads();  // every read of slot_key above precedes the registrations
    if (copied) {
      a.tab.slot_key[base + tid] = key0 + tid;
      a.tab.key2slot[key0 + tid] = base + tid;
    }
    if (tid == 0) {
      *a.tab.clock = clk + uint64_t(u) + uint64_t(P);
      *a.tab.lru_cur = cur ^ 1;
    }
    __syncthreads();
  }

  // ---- 5. victims and recency update in one pass over the recency order.
  // An entry is eligible unless it holds a hit of this wave; the first m_str
  // eligible entries are the victims, the other eligible entries keep their
  // order, and the touched slots (hits and streamed misses) follow in order of
  // their expert's last pair.  The new order goes to the other buffer.
  if (decode) {
    int32_t* lru_out = a.tab.lru[cur ^ 1];
    int neli = 0;
    auto take = [&](bool valid, int s, int oldk, bool have_old) {
      const bool elig = valid && !((sm.prot[s >> 5] >> (s & 31)) & 1u);
      int tot;
      const int vp = neli + block_excount(elig, sm.wbuf, par, &tot);
      if (elig) {
        if (vp < m_str) {
          const int d = sm.sm[vp];
          const int e = sm.D[d];
          const int old = have_old ? oldk : a.tab.slot_key[s];
          if (old >= 0) {
            a.tab.key2slot[old] = -1;
            atomicAdd(&sm.scal[1], 1);
          }
          a.tab.slot_key[s] = key0 + e;
          a.tab.key2slot[key0 + e] = s;
          sm.dslot[d] = s;
        } else {
          lru_out[vp - m_str] = s;
        }
      }
      neli += tot;
    };
#pragma unroll
    for (int j = 0; j < kPf; ++j)
      if (j * NT < C) take(j * NT + tid < C, pf_s[j], pf_key[j], true);
    for (int c0 = kPf * NT; c0 < C; c0 += NT) {
      const int i = c0 + tid;
      take(i < C, i < C ? lru_in[i] : 0, 0, false);
    }
    __syncthreads();
    const int nkeep = neli - m_str;
    // rank of a touched slot = touched experts whose last pair comes earlier
    if (lp) {
      const int nwords = (P + 31) / 32;  // <= 64
      if (tid < nwords) sm.lastbits[tid] = 0u;
      __syncthreads();
      if (tid < nD && sm.cls[tid] != FT_PAIR_MISS_CPU) {
        const int ml = sm.last[sm.D[tid]];
        atomicOr(&sm.lastbits[ml >> 5], 1u << (ml & 31));
      }
      __syncthreads();
      if (wid == 0) {
        const int pc = lane < nwords ? __popc(sm.lastbits[lane]) : 0;
        int x = pc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(x, off, 64);
          if (lane >= off) x += y;
        }
        if (lane < nwords) sm.lastpre[lane] = x - pc;
      }
      __syncthreads();
      if (tid < nD && sm.cls[tid] != FT_PAIR_MISS_CPU) {
        const int ml = sm.last[sm.D[tid]];
        const int rank = sm.lastpre[ml >> 5] + __popc(sm.lastbits[ml >> 5] & ((1u << (ml & 31)) - 1u));
        lru_out[nkeep + rank] = sm.dslot[tid];
        a.tab.slot_last[sm.dslot[tid]] = clk + uint64_t(ml);
      }
    } else {
      for (int d = tid; d < nD; d += NT) {
        if (sm.cls[d] == FT_PAIR_MISS_CPU) continue;
        const int mylast = sm.last[sm.D[d]];
        int rank = 0;
        for (int d2 = 0; d2 < nD; ++d2)
          if (sm.cls[d2] != FT_PAIR_MISS_CPU && sm.last[sm.D[d2]] < mylast) ++rank;
        lru_out[nkeep + rank] = sm.dslot[d];
        a.tab.slot_last[sm.dslot[d]] = clk + uint64_t(mylast);
      }
    }
    if (tid == 0) {
      *a.tab.clock = clk + uint64_t(P);
      *a.tab.lru_cur = cur ^ 1;
    }
    __syncthreads();
  }

  // ---- 7. per-pair decisions (k_stage_rows makes them for staged calls
  // spread over workgroups)
  for (int i = tid; i < (agg ? 0 : P); i += NT) {
    const int d = sm.dix[SEL(i)];
    const int c = sm.cls[d];
    a.pair_flag[pb + i] = uint8_t(c);
    a.pair_slot[pb + i] = c == FT_PAIR_MISS_CPU ? -1 : sm.dslot[d];
  }

  // ---- 8. rank of each pair inside its group (pair order), via ballot match
  int nbits = 1;
  while ((1 << nbits) < nD) ++nbits;
  for (int c0 = 0; c0 < (agg ? 0 : P); c0 += NT) {
    for (int j = tid; j < NW * nD; j += NT) sm.wcnt[j / nD][j % nD] = 0;
    __syncthreads();
    const int i = c0 + tid;
    const bool valid = i < P;
    const int d = valid ? sm.dix[SEL(i)] : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (d >> b) & 1;
      const uint64_t bb = __ballot(valid && bit);
      same &= bit ? bb : ~bb;
    }
    const int lrank = __popcll(same & ((1ull << lane) - 1ull));
    if (valid && lrank == 0) sm.wcnt[wid][d] = __popcll(same);
    __syncthreads();
    for (int g = tid; g < nD; g += NT) {
      int run = sm.cnt[g];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = sm.wcnt[w][g];
        sm.wcnt[w][g] = run;
        run += c;
      }
      sm.cnt[g] = run;
    }
    __syncthreads();
    if (valid) {
      if (lp)
        sm.prow[i] = sm.wcnt[wid][d] + lrank;
      else
        a.pair_row[pb + i] = sm.wcnt[wid][d] + lrank;
    }
    __syncthreads();
  }

  // ---- 9. group offsets and rows
  {
    int tot;
    const int o = block_exscan(tid < nD ? sm.cnt[tid] : 0, sm.wbuf, par, &tot);
    if (tid < nD) sm.off[tid] = o;
  }
  // run-list positions: hits [+ the shared expert], streamed, host
  int nHit;
  const bool ishit = tid < nD && sm.cls[tid] == FT_PAIR_HIT;
  const int hp = block_excount(ishit, sm.wbuf, par, &nHit);
  const bool shared = a.shared_ptr != 0;
  const int n_hit_list = nHit + (shared ? 1 : 0);
  if (tid < nD) sm.gpos[tid] = ishit ? hp : n_hit_list + sm.mpos[tid];
  // prefill: row tiles of the MX GEMM work list, groups in D order, then the
  // shared expert's; a row's slot there is (its tile) * tile_rows + (row in tile)
  int ntiles_d = 0;
  if (a.tiles != nullptr) {
    const int tr = a.tile_rows;
    const int base = block_exscan(tid < nD ? (sm.cnt[tid] + tr - 1) / tr : 0, sm.wbuf, par, &ntiles_d);
    if (tid < nD) sm.tbase[tid] = base;
  }
  __syncthreads();
  // rows; the tokens of a group's first kGroupTok rows also go into its
  // run-list entry, where a decode FFN reads them with the descriptor (the
  // descriptor's other fields are written below, field by field, so the two
  // writes never overlap)
  for (int i = tid; i < (agg ? 0 : P); i += NT) {
    const int d = sm.dix[SEL(i)];
    const int r = lp ? sm.prow[i] : a.pair_row[pb + i];
    const int row = sm.off[d] + r;
    a.pair_row[pb + i] = row;
    a.row_tok[row] = t0 + i / k;
    a.row_w[row] = lp ? sm.pw[i] : a.w[pb + i];
    if (r < kGroupTok) a.gdesc[sm.gpos[d]].tok[r] = uint16_t(t0 + i / k);
    if (a.tiles != nullptr) a.row_slot[row] = (sm.tbase[d] + r / a.tile_rows) * a.tile_rows + r % a.tile_rows;
  }
  if (shared) {
    for (int tt = tid; tt < ntok; tt += NT) {
      a.row_tok[P + tt] = t0 + tt;
      a.row_w[P + tt] = 1.0f;
      if (tt < kGroupTok) a.gdesc[nHit].tok[tt] = uint16_t(t0 + tt);
      if (a.tiles != nullptr) a.row_slot[P + tt] = (ntiles_d + tt / a.tile_rows) * a.tile_rows + tt % a.tile_rows;
    }
  }

  // per-expert results for k_stage_rows: row base, run-list position, class,
  // slot, first MX tile
  if (agg && tid < nD) {
    int32_t* etab = a.agg + 4 * int64_t(a.nchunks) * E + 5 * int64_t(sm.D[tid]);
    etab[0] = sm.off[tid];
    etab[1] = sm.gpos[tid];
    etab[2] = sm.cls[tid];
    etab[3] = sm.cls[tid] == FT_PAIR_MISS_CPU ? -1 : sm.dslot[tid];
    etab[4] = a.tiles != nullptr ? sm.tbase[tid] : 0;
  }

  // ---- 10. group descriptors and run lists
  if (tid < nD) {
    const int c = sm.cls[tid];
    const uint64_t wptr = c == FT_PAIR_MISS_CPU ? 0ull : a.arena + uint64_t(sm.dslot[tid]) * uint64_t(a.slot_bytes);
    const int slot = c == FT_PAIR_MISS_CPU ? -1 : sm.dslot[tid];
    put_desc_head(a.groups[tid], wptr, sm.off[tid], sm.cnt[tid], sm.D[tid], slot);
    const int pos = sm.gpos[tid];
    a.glist[pos] = tid;
    put_desc_head(a.gdesc[pos], wptr, sm.off[tid], sm.cnt[tid], sm.D[tid], slot);
  }
  if (tid == 0 && shared) {
    put_desc_head(a.groups[nD], a.shared_ptr, P, ntok, E, -2);
    a.glist[nHit] = nD;
    put_desc_head(a.gdesc[nHit], a.shared_ptr, P, ntok, E, -2);
  }
  double g = __builtin_inf();
  for (int tt = tid; tt < ntok; tt += NT) g = fmin(g, lp ? sm.pgap[tt] : a.gap[t0 + tt]);
  const bool live_d = tid < nD;
  const int cls_d = live_d ? sm.cls[tid] : -1;
  const int cnt_d = live_d ? sm.cnt[tid] : 0;
  const Closing cl = block_closing(cls_d == FT_PAIR_MISS_CPU ? cnt_d : 0, cls_d == FT_PAIR_HIT ? cnt_d : 0,
                                   cls_d == FT_PAIR_MISS_STREAM ? cnt_d : 0, cnt_d, g, sm.ired, sm.dred);
  // staged calls: experts of the layer resident in the pool (not copied)
  int n_res = 0;
  if (!decode && a.stage_hits) (void)block_excount(tid < E && sm.k2s[tid] >= 0, sm.wbuf, par, &n_res);
  const int max_rows = shared ? max(cl.max_rows, ntok) : cl.max_rows;
  const int cpu_rows = cl.cpu_rows, hit_pairs = cl.hit_pairs, stream_rows = cl.stream_rows;
  const double min_gap = cl.min_gap;
  const int rows = P + (shared ? ntok : 0);

  // prefill: the (group, row tile) work list of the MX GEMM
  if (a.tiles != nullptr) {
    const int tr = a.tile_rows;
    const int nt = live_d ? (cnt_d + tr - 1) / tr : 0;
    const int ntot = ntiles_d;
    const int base = live_d ? sm.tbase[tid] : 0;
    for (int j = 0; j < nt; ++j) {
      a.tiles[2 * (base + j)] = tid;
      a.tiles[2 * (base + j) + 1] = j;
    }
    if (tid == 0) {
      int tot = ntot;
      if (shared) {
        for (int j = 0; j < (ntok + tr - 1) / tr; ++j) {
          a.tiles[2 * tot] = nD;
          a.tiles[2 * tot + 1] = j;
          ++tot;
        }
      }
      a.dev_header[10] = tot;
    }
  }

  if (tid == 0) {
    a.dev_header[0] = t1;
    a.dev_header[1] = nD;
    a.dev_header[2] = n_hit_list;
    a.dev_header[3] = m_str;
    a.dev_header[4] = m_cpu;
    a.dev_header[5] = P;
    a.dev_header[6] = rows;
    a.dev_header[7] = max_rows;
    a.dev_header[8] = cpu_rows;
    a.dev_header[9] = nD + (shared ? 1 : 0);
    // counters: values read in the prologue plus this call's share
    uint64_t d[ST_COUNT] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (decode) {
      d[ST_PAIR_HITS] = uint64_t(hit_pairs);
      d[ST_PAIR_MISSES] = uint64_t(P - hit_pairs);
      d[ST_EXPERT_HITS] = uint64_t(nHit);
      d[ST_EXPERT_MISSES] = uint64_t(nM);
      d[ST_CPU_MISSES] = uint64_t(m_cpu);
      d[ST_EVICTIONS] = uint64_t(sm.scal[1]);
      d[ST_BYTES_H2D] = uint64_t(m_str) * uint64_t(a.expert_bytes) + uint64_t(cpu_rows) * uint64_t(a.hidden) * 2ull;
    } else {
      d[ST_PAIR_HITS] = uint64_t(hit_pairs);
      d[ST_PAIR_MISSES] = uint64_t(P - hit_pairs);
      d[ST_EXPERT_HITS] = uint64_t(n_res);
      d[ST_EXPERT_MISSES] = uint64_t(E - n_res);
      d[ST_BYTES_H2D] = uint64_t(E - n_res) * uint64_t(a.expert_bytes);
    }
    d[ST_CALLS] = t0 == 0 ? 1ull : 0ull;
#pragma unroll
    for (int i = 0; i < ST_COUNT; ++i) st[i] = st0[i] + d[i];
    a.tab.min_gap[a.layer] = fmin(gap0, min_gap);
    if (a.prof_cnt != nullptr) {
      // groups and rows behind the timed stages of this call (the FFN over
      // the hit list and the streamed misses; the copy of the streamed misses)
      const uint64_t g_all = uint64_t(n_hit_list + m_str);
      const uint64_t r_all = uint64_t(hit_pairs + (shared ? ntok : 0) + stream_rows);
#pragma unroll
      for (int st2 = 0; st2 < 3; ++st2) {
        if (!((a.prof_stages >> st2) & 1)) continue;
        uint64_t* c = a.prof_cnt + (st2 * 4 + a.fmt) * 2;
        c[0] = pc0[st2][0] + (st2 == 2 ? uint64_t(m_str) : g_all);
        c[1] = pc0[st2][1] + (st2 == 2 ? 0ull : r_all);
      }
    }
  }

  // ---- 11. host readback (decode): header, miss lists, host-computed rows
  if (a.host_rb != nullptr) {
    ResolveHeader* h = reinterpret_cast<ResolveHeader*>(a.host_rb);
    int32_t* se = reinterpret_cast<int32_t*>(a.host_rb + sizeof(ResolveHeader));
    int32_t* ss = se + E;
    int32_t* ce = ss + E;
    int32_t* cb = ce + E;
    int32_t* cc = cb + E;
    int32_t* ct = cc + E;
    float* cw = reinterpret_cast<float*>(ct + a.T * k);
    if (tid < nD) {
      const int c = sm.cls[tid];
      const int mpv = sm.mpos[tid];
      if (c == FT_PAIR_MISS_STREAM) {
        se[mpv] = sm.D[tid];
        ss[mpv] = sm.dslot[tid];
      } else if (c == FT_PAIR_MISS_CPU) {
        ce[mpv - m_str] = sm.D[tid];
        cb[mpv - m_str] = sm.off[tid];
        cc[mpv - m_str] = sm.cnt[tid];
      }
    }
    if (m_cpu > 0) {
      // rows of host-computed groups, packed group after group: the groups'
      // D indices and packed bases in LDS (first[] and tbase[] are free in
      // decode calls by now; the lists above are in host memory, which the
      // device does not read back)
      if (tid < nD && sm.cls[tid] == FT_PAIR_MISS_CPU) sm.first[sm.mpos[tid] - m_str] = tid;
      __syncthreads();
      int tot;
      const int hb = block_exscan(tid < m_cpu ? sm.cnt[sm.first[tid]] : 0, sm.wbuf, par, &tot);
      if (tid < m_cpu) sm.tbase[tid] = hb;
      __syncthreads();
      for (int idx = tid; idx < cpu_rows; idx += NT) {
        int lo = 0, hi = m_cpu - 1;  // last group whose base is <= idx
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sm.tbase[mid] <= idx) lo = mid;
          else hi = mid - 1;
        }
        const int row = sm.off[sm.first[lo]] + (idx - sm.tbase[lo]);
        ct[idx] = a.row_tok[row];
        cw[idx] = a.row_w[row];
      }
    }
    if (tid == 0) {
      h->t1 = t1;
      h->n_groups = nD;
      h->n_hit_list = n_hit_list;
      h->n_stream = m_str;
      h->n_cpu = m_cpu;
      h->pairs = P;
      h->rows = rows;
      h->max_rows = max_rows;
      h->cpu_rows = cpu_rows;
      h->rows_hit_list = hit_pairs + (shared ? ntok : 0);
      h->rows_stream = stream_rows;
      h->min_gap = min_gap;
    }
    if (a.host_wait) {
      // the host spins on the stamp: publish everything above first
      __threadfence_system();
      __syncthreads();
      if (tid == 0) __hip_atomic_store(&h->seq, uint32_t(a.stamp), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// Staged calls spread over workgroups, 1: per chunk of kStageChunk pairs, each
// expert's pair count and first and last pair.
__global__ __launch_bounds__(NT) void k_stage_hist(const int32_t* __restrict__ sel, int P, int E,
                                                   int32_t* __restrict__ agg, int nchunks) {
  __shared__ int cnt[kMaxExperts], first[kMaxExperts], last[kMaxExperts];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < E; e += NT) {
    cnt[e] = 0;
    first[e] = 0x7fffffff;
    last[e] = -1;
  }
  __syncthreads();
  const int i = c * kStageChunk + tid;
  if (i < P) {
    const int e = sel[i];
    atomicAdd(&cnt[e], 1);
    atomicMin(&first[e], i);
    atomicMax(&last[e], i);
  }
  __syncthreads();
  int32_t* hist = agg + int64_t(c) * E;
  for (int e = tid; e < E; e += NT) {
    hist[e] = cnt[e];
    hist[int64_t(nchunks) * E + e] = first[e];
    hist[2 * int64_t(nchunks) * E + e] = last[e];
  }
}

// Staged calls spread over workgroups, 3 (after the resolve kernel): the
// pairs of one chunk -- flag, slot and row of each pair (its group's row base
// + the pairs of its expert in earlier chunks + its rank in this chunk, by a
// wavefront-ballot match and a per-wave prefix), the row's token and weight,
// the group's first tokens in its run-list entry and the row's MX tile slot.
__global__ __launch_bounds__(NT) void k_stage_rows(ResolveArgs a) {
  __shared__ int wcnt[NW][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, c = blockIdx.x;
  const int E = a.E, k = a.k, P = a.T * a.k;
  const int32_t* cbase = a.agg + 3 * int64_t(a.nchunks) * E + int64_t(c) * E;
  const int32_t* etab = a.agg + 4 * int64_t(a.nchunks) * E;
  for (int j = tid; j < NW * E; j += NT) wcnt[j / E][j % E] = 0;
  __syncthreads();
  const int i = c * kStageChunk + tid;
  const bool valid = i < P;
  const int e = valid ? a.sel[i] : 0;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    same &= bit ? bb : ~bb;
  }
  const int lrank = __popcll(same & ((1ull << lane) - 1ull));
  if (valid && lrank == 0) wcnt[wid][e] = __popcll(same);
  __syncthreads();
  for (int g = tid; g < E; g += NT) {
    int run = cbase[g];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int v = wcnt[w][g];
      wcnt[w][g] = run;
      run += v;
    }
  }
  __syncthreads();
  if (!valid) return;
  const int r = wcnt[wid][e] + lrank;  // rank in the group
  const int32_t* et = etab + 5 * e;
  const int row = et[0] + r, cls = et[2];
  a.pair_flag[i] = uint8_t(cls);
  a.pair_slot[i] = et[3];
  a.pair_row[i] = row;
  a.row_tok[row] = i / k;
  a.row_w[row] = a.w[i];
  if (r < kGroupTok) a.gdesc[et[1]].tok[r] = uint16_t(i / k);
  if (a.tiles != nullptr) a.row_slot[row] = (et[4] + r / a.tile_rows) * a.tile_rows + r % a.tile_rows;
}

// Free slots (prefill staging halves, or slots whose copy failed) and restore
// the recency order invariant: free slots first by index, then residents in
// their previous order.
__global__ __launch_bounds__(NT) void k_free_slots(DevTable tab, int C, int lo0, int hi0, int lo1, int hi1,
                                                   const int32_t* keys, const int32_t* slots, int n,
                                                   uint64_t* evict_stat) {
  __shared__ int wbuf[2][NW];
  __shared__ int nev;
  int par = 0;
  const int tid = threadIdx.x;
  if (tid == 0) nev = 0;
  __syncthreads();
  for (int s = tid; s < C; s += NT) {
    const bool in = (s >= lo0 && s < hi0) || (s >= lo1 && s < hi1);
    if (in) {
      const int old = tab.slot_key[s];
      if (old >= 0) {
        tab.key2slot[old] = -1;
        tab.slot_key[s] = -1;
        atomicAdd(&nev, 1);
      }
    }
  }
  for (int i = tid; i < n; i += NT) {
    const int s = slots[i];
    if (tab.slot_key[s] == keys[i]) {
      tab.slot_key[s] = -1;
      tab.key2slot[keys[i]] = -1;
    }
  }
  __syncthreads();
  const int cur = *tab.lru_cur;
  const int32_t* lru_in = tab.lru[cur];
  int32_t* lru_out = tab.lru[cur ^ 1];
  int nfree = 0;
  for (int c0 = 0; c0 < C; c0 += NT) {
    const int s = c0 + tid;
    const bool f = s < C && tab.slot_key[s] < 0;
    int tot;
    const int p = block_excount(f, wbuf, par, &tot);
    if (f) lru_out[nfree + p] = s;
    nfree += tot;
  }
  int nres = 0;
  for (int c0 = 0; c0 < C; c0 += NT) {
    const int i = c0 + tid;
    int s = 0;
    bool r = false;
    if (i < C) {
      s = lru_in[i];
      r = tab.slot_key[s] >= 0;
    }
    int tot;
    const int p = block_excount(r, wbuf, par, &tot);
    if (r) lru_out[nfree + nres + p] = s;
    nres += tot;
  }
  __syncthreads();
  if (tid == 0) {
    *tab.lru_cur = cur ^ 1;
    if (evict_stat) *evict_stat += uint64_t(nev);
  }
}

}  // namespace

// Staged calls (a.agg set; one wave starting at token 0) run as three
// kernels: per-chunk histograms over many workgroups, the resolve itself on
// per-expert totals, the per-pair rows over many workgroups.  The results
// are the same as the one-workgroup resolve's.  The events bracket all three.
hipError_t launch_resolve(const ResolveArgs& a, hipStream_t s, Ev ev) {
  if (a.agg == nullptr) {
    ft_launch(k_resolve, dim3(1), dim3(NT), s, ev, a);
    return hipGetLastError();
  }
  const int P = a.T * a.k;
  ft_launch(k_stage_hist, dim3(a.nchunks), dim3(NT), s, Ev{ev.a, nullptr}, a.sel, P, a.E, a.agg, a.nchunks);
  ft_launch(k_resolve, dim3(1), dim3(NT), s, Ev{}, a);
  ft_launch(k_stage_rows, dim3(a.nchunks), dim3(NT), s, Ev{nullptr, ev.b}, a);
  return hipGetLastError();
}

hipError_t launch_stage_table(DevTable tab, int E, int C, int layer, int num_layers, int pairs,
                              int64_t expert_bytes, hipStream_t s) {
  (void)pairs;
  (void)expert_bytes;
  const int h0 = layer & 1;
  const int lo0 = h0 * E, hi0 = lo0 + E;
  int lo1 = 0, hi1 = 0;
  if (layer + 1 < num_layers) {
    lo1 = ((layer + 1) & 1) * E;
    hi1 = lo1 + E;
  }
  hipLaunchKernelGGL(k_free_slots, dim3(1), dim3(NT), 0, s, tab, C, lo0, hi0, lo1, hi1, nullptr, nullptr, 0,
                     tab.stats + int64_t(layer) * ST_COUNT + ST_EVICTIONS);
  return hipGetLastError();
}

hipError_t launch_uncommit(DevTable tab, const int32_t* keys, const int32_t* slots, int n, int C,
                           hipStream_t s) {
  hipLaunchKernelGGL(k_free_slots, dim3(1), dim3(NT), 0, s, tab, C, 0, 0, 0, 0, keys, slots, n, nullptr);
  return hipGetLastError();
}

}  // namespace ftmoe
