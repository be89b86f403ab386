// On-GPU redundant-expert planner for gfx950.
//
// Plans a few duplicated experts from the current router output so that every
// rank receives exactly S*K token-slots, and gives every slot its place in its
// rank's static S*K buffer [ai-maestro.online "Moonshot AI open-sources MoonEP",
// sections "The core idea: dynamic redundant experts" and "The memory
// contract"]. The pages fix only the invariants; the rule implemented is stated
// in moonep.h (moonep_plan). Four launches, no host synchronisation (on layers of at
// most kFusedMaxChunks chunks, count, scan and solve share one launch: see
// plan_count_solve_kernel):
//
//   count   one wavefront per chunk of 64 tokens: per-chunk expert histogram
//           (LDS atomics) into counts[chunk][E]; flags bad or repeated ids.
//   scan    column-wise exclusive prefix of counts over the chunks of each
//           partition of kScanPart chunks, and the partition totals.
//           (The solve kernel folds the partition totals into T[e] and a
//           prefix over partitions; assign adds that prefix: together the base
//           rank of each chunk's first slot of every expert.)
//   solve   one workgroup: rank loads, donor tree, per-donor expert layout,
//           pieces, prefetch slots, cu_seqlens and a per-expert piece table
//           (first rank t and destination base of every piece).
//   assign  one wavefront per chunk again: the stable rank t of every slot
//           within its expert = chunk base + rank among equal ids in earlier
//           64-slot steps (LDS counter) + rank among equal ids in the same step
//           (wavefront match built from ballots); then slot_map / src_index.
#include "common.h"

namespace moonep {

constexpr int kWavesPerBlock = 4;
constexpr int kSolveThreads = 1024;

// Inclusive scan across the 64 lanes of a wavefront with DPP (no LDS round trips):
// Hillis-Steele over row shifts of 1, 2, 4 and 8 lanes builds the prefix inside each
// 16-lane row (lanes shifted in from outside the row read 0); then lane 15's total is
// broadcast into rows 1 and 3, and lane 31's into rows 2 and 3.
__device__ inline int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2, 3
  return v;
}

// Sum over a wavefront whose 64 lanes are all active: lane 63 of the inclusive scan,
// read into a scalar register (no LDS round trip).
__device__ inline int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_incl_scan(v), 63); }

// Exclusive scan across one wavefront (all 64 lanes active); *total gets the sum.
__device__ inline int wave_excl_scan(int v, int* total) {
  const int incl = wave_incl_scan(v);
  *total = __builtin_amdgcn_readlane(incl, 63);
  return incl - v;
}

// Exclusive scan across a 1024-thread block; *total gets the block sum.
__device__ inline int block_excl_scan(int v, int* swave, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) swave[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int x = lane < kSolveThreads / 64 ? swave[lane] : 0;
    const int xi = wave_incl_scan(x);
    if (lane < kSolveThreads / 64) swave[lane] = xi - x;
    if (lane == kSolveThreads / 64 - 1) swave[kSolveThreads / 64] = xi;
  }
  __syncthreads();
  const int r = swave[w] + incl - v;
  *total = swave[kSolveThreads / 64];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- count
// One token's K expert ids into an LDS histogram; returns the error bits it finds. The
// ids are loaded 8 at a time, all 8 loads in flight together.
__device__ inline int count_token(const int32_t* row, int K, int E, int32_t* hist) {
  int err = 0;
  for (int k0 = 0; k0 < K; k0 += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = k0 + i < K ? row[k0 + i] : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = v[i];
      if (k0 + i >= K) break;
      if (e < 0 || e >= E) {
        err |= MOONEP_ERR_ID_RANGE;
        continue;
      }
      for (int k2 = 0; k2 < k0; ++k2)  // ids of earlier batches (K > 8 only)
        if (row[k2] == e) err |= MOONEP_ERR_ID_DUP;
#pragma unroll
      for (int j = 0; j < i; ++j)
        if (v[j] == e) err |= MOONEP_ERR_ID_DUP;
      atomicAdd(&hist[e], 1);
    }
  }
  return err;
}

__global__ __launch_bounds__(256) void plan_count_kernel(const int32_t* __restrict__ topk, int N,
                                                         int K, int E, int nchunk,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ flags) {
  extern __shared__ int32_t lds[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int32_t* hist = lds + w * E;
  for (int e = lane; e < E; e += 64) hist[e] = 0;
  __syncthreads();
  const int c = blockIdx.x * kWavesPerBlock + w;
  const int g = c * kChunkTokens + lane;
  const int err = c < nchunk && g < N ? count_token(topk + int64_t(g) * K, K, E, hist) : 0;
  __syncthreads();
  if (c < nchunk)
    for (int e = lane; e < E; e += 64) counts[int64_t(c) * E + e] = hist[e];
  if (err) atomicOr(&flags[kFlagError], err);
}

// ---------------------------------------------------------------- scan
// Block (column group, partition): 64 experts (lanes) x 16 wavefronts of
// kScanPart / 16 chunks each, one round of independent loads per wavefront.
// counts[c][e] becomes the exclusive prefix over the partition's chunks before c;
// part[p][e] the partition total.
constexpr int kScanPerWave = kScanPart / 16;

__global__ __launch_bounds__(1024) void plan_scan_kernel(int32_t* __restrict__ counts, int nchunk,
                                                         int E, int32_t* __restrict__ part) {
  __shared__ int32_t wsum[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int c0 = blockIdx.y * kScanPart + w * kScanPerWave;
  const bool col = e < E;
  int v[kScanPerWave];
#pragma unroll
  for (int i = 0; i < kScanPerWave; ++i)
    v[i] = (col && c0 + i < nchunk) ? counts[int64_t(c0 + i) * E + e] : 0;
  int s = 0;
#pragma unroll
  for (int i = 0; i < kScanPerWave; ++i) {
    const int x = v[i];
    v[i] = s;
    s += x;
  }
  wsum[w][lane] = s;
  __syncthreads();
  if (w == 0) {
    int run = 0;
    for (int i = 0; i < 16; ++i) {
      const int x = wsum[i][lane];
      wsum[i][lane] = run;
      run += x;
    }
    if (col) part[int64_t(blockIdx.y) * E + e] = run;
  }
  __syncthreads();
  const int off = wsum[w][lane];
#pragma unroll
  for (int i = 0; i < kScanPerWave; ++i)
    if (col && c0 + i < nchunk) counts[int64_t(c0 + i) * E + e] = off + v[i];
}

// ---------------------------------------------------------------- solve
struct SolveArgs {
  int R, S, E, K, B, G, SK;
  int64_t NK;
  int32_t* part;      // [npart, E] partition totals -> exclusive prefix over partitions
  int npart;
  int32_t* cu;        // [R, E+B+1]
  int32_t* replica;   // [R, B]
  int32_t* piece_ptr, *piece_tlo, *piece_base;
  int32_t* flags;
};

// LDS carve-up of the solve kernel (ints).
struct SolveLds {
  int T, seqpos, off, seq, npiece, hot, hsum, crank, csum, cdon, cfirst, clast, chain, L, gchild,
      gamt, glo, gfirst, dptr, homestart, rowlen, swave, misc, total;
  __host__ __device__ SolveLds(int R, int E, int B) {
    int o = 0;
    T = o; o += E;
    seqpos = o; o += E;
    off = o; o += E;
    seq = o; o += E;
    npiece = o; o += E;
    hot = o; o += R;      // hot ranks in ascending id
    hsum = o; o += R;     // their excess, inclusive prefix
    crank = o; o += R;    // cold ranks in ascending id
    csum = o; o += R;     // their need, inclusive prefix
    cdon = o; o += R;     // hot index each cold rank takes from
    cfirst = o; o += R;   // per hot index: first and last cold index it gives to
    clast = o; o += R;
    chain = o; o += R;    // per hot index: what it passes to the previous hot rank
    L = o; o += R;
    gchild = o; o += R;
    gamt = o; o += R;
    glo = o; o += R;
    gfirst = o; o += R;
    dptr = o; o += R + 1;
    homestart = o; o += R;
    rowlen = o; o += R * (E + B);
    swave = o; o += kSolveThreads / 64 + 1;
    misc = o; o += 8;
    total = o;
  }
};

// Intersect expert e's layout interval with donor p's gift ranges and home tail.
// Calls f(dest_rank, row, t_lo, t_hi) for each non-empty piece in t order.
template <typename F>
__device__ inline void for_each_piece(const SolveArgs& a, const int* sm, const SolveLds& L, int e,
                                      F&& f) {
  const int p = e / a.G;
  const int off = sm[L.off + e], t = sm[L.T + e];
  for (int gi = sm[L.dptr + p]; gi < sm[L.dptr + p + 1]; ++gi) {
    const int lo = sm[L.glo + gi], hi = lo + sm[L.gamt + gi];
    const int x = max(lo, off), y = min(hi, off + t);
    if (x < y) {
      const int j = sm[L.seqpos + e] - sm[L.gfirst + gi];
      const int row = j < a.B ? a.E + j : e;  // j >= B: overflow, home row in place
      f(sm[L.gchild + gi], row, x - off, y - off, j);
    }
  }
  const int x = max(sm[L.homestart + p], off), y = min(sm[L.L + p], off + t);
  if (x < y) f(p, e, x - off, y - off, -1);
}

// The donor tree of the solve kernel (rule and closed form where it is called). Run by
// the whole block (scan and sync across all threads) or, when R <= 64, by one wavefront
// alone: the same steps with wavefront scans and no block barriers.
template <class Scan, class Sync>
__device__ inline void donor_tree(const SolveArgs& a, int* sm, const SolveLds& L, int tid,
                                  Scan scan, Sync sync) {
  const int p = tid;
  const bool in = p < a.R;
  const int lp = in ? sm[L.L + p] : 0;
  const int ishot = in && lp > a.SK, iscold = in && lp < a.SK;
  int nhot, ncold, sx, sn;
  const int hidx = scan(ishot, &nhot);
  const int cidx = scan(iscold, &ncold);
  const int hpre = scan(ishot ? lp - a.SK : 0, &sx);
  const int cpre = scan(iscold ? a.SK - lp : 0, &sn);
  if (ishot) {
    sm[L.hot + hidx] = p;
    sm[L.hsum + hidx] = hpre + (lp - a.SK);
    sm[L.cfirst + hidx] = -1;
    sm[L.clast + hidx] = -2;
  }
  if (iscold) {
    sm[L.crank + cidx] = p;
    sm[L.csum + cidx] = cpre + (a.SK - lp);
  }
  sync();
  // cold j: its donor's hot index, by binary search over S
  if (tid < ncold) {
    const int dprev = tid > 0 ? sm[L.csum + tid - 1] : 0;
    int lo = 0, hi = nhot - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sm[L.hsum + mid] > dprev) hi = mid; else lo = mid + 1;
    }
    sm[L.cdon + tid] = lo;
  }
  // hot i >= 1: the gift to hot i-1, by binary search over D
  if (tid < nhot) {
    int amt = 0;
    if (tid > 0) {
      const int sp = sm[L.hsum + tid - 1];
      int lo = 0, hi = ncold;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sm[L.csum + mid] > sp) hi = mid; else lo = mid + 1;
      }
      const int dprev = lo > 0 ? sm[L.csum + lo - 1] : 0;
      if (lo < ncold && dprev < sp) amt = sm[L.csum + lo] - sp;
    }
    sm[L.chain + tid] = amt;
  }
  sync();
  // the run of cold ranks each donor gives to (cdon is non-decreasing in j)
  if (tid < ncold) {
    const int d = sm[L.cdon + tid];
    if (tid == 0 || sm[L.cdon + tid - 1] != d) sm[L.cfirst + d] = tid;
    if (tid == ncold - 1 || sm[L.cdon + tid + 1] != d) sm[L.clast + d] = tid;
  }
  sync();
  // gift counts per donor rank, grouped by donor in ascending id
  int cnt = 0, chain_amt = 0, first = -1, last = -2;
  if (ishot) {
    chain_amt = sm[L.chain + hidx];
    first = sm[L.cfirst + hidx];
    last = sm[L.clast + hidx];
    cnt = (chain_amt > 0) + (last - first + 1);
  }
  int ngift;
  const int base = scan(cnt, &ngift);
  if (in) sm[L.dptr + p] = base;
  if (tid == 0) {
    sm[L.dptr + a.R] = ngift;
    sm[L.misc] = ngift;
  }
  if (in) {
    int given = 0;
    if (ishot) {
      const int d0 = first > 0 ? sm[L.csum + first - 1] : 0;
      given = chain_amt + (last >= first ? sm[L.csum + last] - d0 : 0);
      if (chain_amt > 0) {
        sm[L.gchild + base] = sm[L.hot + hidx - 1];
        sm[L.gamt + base] = chain_amt;
        sm[L.glo + base] = 0;
      }
    }
    sm[L.homestart + p] = given;
  }
  sync();
  if (tid < ncold) {
    const int i = sm[L.cdon + tid];
    const int d = sm[L.hot + i];
    const int ch = sm[L.chain + i];
    const int first_j = sm[L.cfirst + i];
    const int k = sm[L.dptr + d] + (ch > 0) + (tid - first_j);
    const int dprev = tid > 0 ? sm[L.csum + tid - 1] : 0;
    const int dfirst = first_j > 0 ? sm[L.csum + first_j - 1] : 0;
    sm[L.gchild + k] = sm[L.crank + tid];
    sm[L.gamt + k] = sm[L.csum + tid] - dprev;
    sm[L.glo + k] = ch + (dprev - dfirst);
  }
}

// The solve step, run by one workgroup of kSolveThreads threads over the LDS area `sm`
// (SolveLds(R, E, B).total ints).
__device__ __forceinline__ void solve_plan(const SolveArgs& a, int* sm) {
  const SolveLds L(a.R, a.E, a.B);
  const int tid = threadIdx.x;
  const int EB = a.E + a.B;

  __shared__ unsigned int s_total;
  if (tid == 0) s_total = 0;
  __syncthreads();
  // T[e]: sum of the partition totals, which become the prefix over partitions
  unsigned int sum = 0;   // at most N*K < 2^31: every slot counts once, and only valid ids
  for (int e = tid; e < a.E; e += kSolveThreads) {
    int run = 0;
    for (int p0 = 0; p0 < a.npart; p0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = p0 + i < a.npart ? a.part[int64_t(p0 + i) * a.E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (p0 + i < a.npart) a.part[int64_t(p0 + i) * a.E + e] = run;
        run += v[i];
      }
    }
    sm[L.T + e] = run;
    sum += run;
  }
  sum = unsigned(wave_sum(int(sum)));  // below 2^31: a wavefront's share of N*K
  if ((tid & 63) == 0 && sum) atomicAdd(&s_total, sum);
  for (int i = tid; i < a.R * EB; i += kSolveThreads) sm[L.rowlen + i] = 0;
  for (int i = tid; i < a.R * a.B; i += kSolveThreads) a.replica[i] = -1;
  __syncthreads();

  if (s_total != (unsigned int)a.NK) {  // an id outside [0,E): publish an empty plan
    for (int i = tid; i < a.R * (EB + 1); i += kSolveThreads) a.cu[i] = 0;
    for (int i = tid; i <= a.E; i += kSolveThreads) a.piece_ptr[i] = 0;
    if (tid == 0) a.flags[kFlagPlanValid] = 0;
    return;
  }

  // rank loads L_p, and each group's layout: an expert's position by (T desc, e asc) is
  // the number of its group's experts that sort before it
  if (a.G <= 64) {
    // a wavefront per group, a lane per expert: the load by a shuffle reduction, the
    // positions by one pass over the group's T read lane by lane
    const int lane = tid & 63, w = tid >> 6;
    for (int p = w; p < a.R; p += kSolveThreads / 64) {
      const int e = p * a.G + lane;
      const int te = lane < a.G ? sm[L.T + e] : 0;
      const int s = wave_sum(te);
      if (lane == 0) sm[L.L + p] = s;
      int pos = 0;
      for (int j = 0; j < a.G; ++j) {
        const int tj = __builtin_amdgcn_readlane(te, j);
        pos += (tj > te) || (tj == te && j < lane);
      }
      if (lane < a.G) {
        sm[L.seqpos + e] = pos;
        sm[L.seq + p * a.G + pos] = e;
      }
    }
  } else {
    for (int p = tid; p < a.R; p += kSolveThreads) {
      int s = 0;
      for (int e = p * a.G; e < (p + 1) * a.G; ++e) s += sm[L.T + e];
      sm[L.L + p] = s;
    }
    for (int e = tid; e < a.E; e += kSolveThreads) {
      const int p = e / a.G, te = sm[L.T + e];
      int pos = 0;
      for (int e2 = p * a.G; e2 < (p + 1) * a.G; ++e2) {
        const int t2 = sm[L.T + e2];
        pos += (t2 > te) || (t2 == te && e2 < e);
      }
      sm[L.seqpos + e] = pos;
      sm[L.seq + p * a.G + pos] = e;
    }
  }
  __syncthreads();
  // off(e): T summed over the experts before e in its group's layout, one
  // wavefront-wide exclusive scan per group and 64 layout positions
  {
    const int lane = tid & 63, w = tid >> 6;
    for (int p = w; p < a.R; p += kSolveThreads / 64) {
      int carry = 0;
      for (int b = 0; b < a.G; b += 64) {
        const int s = b + lane;
        const int e = s < a.G ? sm[L.seq + p * a.G + s] : 0;
        const int t = s < a.G ? sm[L.T + e] : 0;
        const int incl = wave_incl_scan(t);
        if (s < a.G) sm[L.off + e] = carry + incl - t;
        carry += __builtin_amdgcn_readlane(incl, 63);
      }
    }
  }

  // Donor tree, in closed form. The rule (moonep_plan) walks the cold ranks in
  // ascending id; a receiver takes all it lacks from the current donor, a donor
  // that runs short takes the deficit from the next hot rank. With S_i the hot
  // ranks' excess summed in ascending id (inclusive) and D_j the cold ranks' need
  // likewise, the donor's running surplus before cold j is S_i - D_(j-1), so:
  //   cold j takes from hot i(j) = min{ i : S_i > D_(j-1) };
  //   hot i gives D_j - S_(i-1) to hot i-1 exactly when D_(j-1) < S_(i-1) < D_j,
  //   and that gift is made before any of hot i's gifts to cold ranks.
  // A donor's gift list is therefore its gift to the previous hot rank (if any),
  // then its cold ranks in ascending id; consecutive layout ranges from 0 follow.
  if (a.R <= 64) {
    if (tid < 64)
      donor_tree(a, sm, L, tid, [](int v, int* t) { return wave_excl_scan(v, t); }, []() {
        // a wavefront's LDS accesses run in program order: keep the compiler from
        // moving them across the steps
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      });
  } else {
    donor_tree(a, sm, L, tid,
               [&](int v, int* t) { return block_excl_scan(v, sm + L.swave, t); },
               []() { __syncthreads(); });
  }
  __syncthreads();

  // layout position of the first expert each gift range touches
  const int ngift = sm[L.misc];
  for (int k = tid; k < ngift; k += kSolveThreads) {
    int d = 0;
    for (int p = 0; p < a.R; ++p)
      if (k >= sm[L.dptr + p] && k < sm[L.dptr + p + 1]) d = p;
    const int lo = sm[L.glo + k];
    int s = 0;
    while (s < a.G - 1) {
      const int e = sm[L.seq + d * a.G + s];
      if (sm[L.off + e] + sm[L.T + e] > lo) break;
      ++s;
    }
    sm[L.gfirst + k] = s;
  }
  __syncthreads();

  // pieces: row lengths, prefetch slots, piece counts
  for (int e = tid; e < a.E; e += kSolveThreads) {
    int n = 0;
    for_each_piece(a, sm, L, e, [&](int q, int row, int tlo, int thi, int j) {
      sm[L.rowlen + q * EB + row] = thi - tlo;
      if (j >= 0 && j < a.B) a.replica[q * a.B + j] = e;
      ++n;
    });
    sm[L.npiece + e] = n;
  }
  __syncthreads();

  // cu_seqlens: exclusive prefix of row lengths per rank; rowlen becomes row start
  {
    const int lane = tid & 63, w = tid >> 6;
    for (int q = w; q < a.R; q += kSolveThreads / 64) {
      int carry = 0;
      if (lane == 0) a.cu[q * (EB + 1)] = 0;
      for (int base = 0; base < EB; base += 64) {
        const int i = base + lane;
        const int v = i < EB ? sm[L.rowlen + q * EB + i] : 0;
        const int incl = wave_incl_scan(v);
        if (i < EB) {
          a.cu[q * (EB + 1) + i + 1] = carry + incl;
          sm[L.rowlen + q * EB + i] = carry + incl - v;
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
      }
    }
  }
  int total_pieces;
  const int my_np = tid < a.E ? sm[L.npiece + tid] : 0;
  const int first = block_excl_scan(my_np, sm + L.swave, &total_pieces);
  if (tid < a.E) sm[L.npiece + tid] = first;  // now the piece pointer
  __syncthreads();

  // piece table: per expert, pieces in t order with dest base = q*SK + row start - t_lo
  for (int e = tid; e < a.E; e += kSolveThreads) {
    int k = sm[L.npiece + e];
    a.piece_ptr[e] = k;
    for_each_piece(a, sm, L, e, [&](int q, int row, int tlo, int thi, int j) {
      a.piece_tlo[k] = tlo;
      a.piece_base[k] = q * a.SK + sm[L.rowlen + q * EB + row] - tlo;
      ++k;
    });
  }
  if (tid == 0) {
    a.piece_ptr[a.E] = total_pieces;
    a.flags[kFlagPlanValid] = 1;
  }
}

__global__ __launch_bounds__(kSolveThreads) void plan_solve_kernel(SolveArgs a) {
  extern __shared__ int sm[];
  solve_plan(a, sm);
}

// ---------------------------------------------------------------- count + scan + solve
// Small layers (at most kFusedMaxChunks chunks): one launch of kSolveThreads-thread
// workgroups, kFusedChunks chunks each, one per wavefront. A workgroup counts its chunks,
// writes each chunk's exclusive prefix over its own earlier chunks into counts and its
// totals into part[blockIdx.x] (a partition of kFusedChunks chunks). The last workgroup
// to finish (an arrival counter after a device-scope fence; no workgroup waits for
// another) then runs the solve step on all of them.
__global__ __launch_bounds__(kSolveThreads) void plan_count_solve_kernel(
    const int32_t* __restrict__ topk, int N, int nchunk, int32_t* __restrict__ counts,
    SolveArgs a) {
  extern __shared__ int sm[];
  __shared__ int s_last;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int E = a.E;
  int32_t* hist = sm + w * E;  // [kFusedChunks][E], then the solve step's area
  for (int e = lane; e < E; e += 64) hist[e] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * kFusedChunks;
  const int c = c0 + w;
  const int g = c * kChunkTokens + lane;
  const int err = c < nchunk && g < N ? count_token(topk + int64_t(g) * a.K, a.K, E, hist) : 0;
  if (err) atomicOr(&a.flags[kFlagError], err);
  __syncthreads();
  for (int e = tid; e < E; e += kSolveThreads) {
    int run = 0;
    for (int i = 0; i < kFusedChunks; ++i) {
      const int x = sm[i * E + e];
      if (c0 + i < nchunk) counts[int64_t(c0 + i) * E + e] = run;
      run += x;
    }
    a.part[int64_t(blockIdx.x) * E + e] = run;
  }
  // The barrier completes the workgroup's stores; one acquire-release counter update
  // then publishes them device-wide and, in the last workgroup, makes every other
  // workgroup's stores visible to the whole workgroup (it shares one L1 and L2).
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&a.flags[kFlagPlanArrive], 1, __ATOMIC_ACQ_REL,
                                    __HIP_MEMORY_SCOPE_AGENT) == int(gridDim.x) - 1;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) a.flags[kFlagPlanArrive] = 0;  // ready for the layer's next plan
  solve_plan(a, sm);
}

// ---------------------------------------------------------------- assign
// The piece table is staged in LDS by the workgroup; each wavefront loads the ids
// of 8 steps at once, so a step waits on no global load.
constexpr int kAssignBatch = 8;

__global__ __launch_bounds__(256) void plan_assign_kernel(
    const int32_t* __restrict__ topk, int N, int K, int E, int nchunk, int nbits,
    const int32_t* __restrict__ base, const int32_t* __restrict__ part, int part_chunks,
    const int32_t* __restrict__ piece_ptr, const int32_t* __restrict__ piece_tlo,
    const int32_t* __restrict__ piece_base, int max_pieces, const int32_t* __restrict__ flags,
    int32_t* __restrict__ slot_map, int32_t* __restrict__ src_index) {
  // LDS: run[kWavesPerBlock][E] | ptr[E+1] | tlo[max_pieces] | pbase[max_pieces]
  extern __shared__ int32_t lds[];
  int32_t* s_ptr = lds + kWavesPerBlock * E;
  int32_t* s_tlo = s_ptr + E + 1;
  int32_t* s_base = s_tlo + max_pieces;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * kWavesPerBlock + w;
  const bool have = c < nchunk;
  const int64_t NK = int64_t(N) * K;
  const int64_t u0 = int64_t(c) * kChunkTokens * K;
  const int64_t u1 = have ? min(NK, u0 + int64_t(kChunkTokens) * K) : u0;
  const int nsteps = int((u1 - u0 + 63) / 64);
  int32_t* run = lds + w * E;  // next rank of every expert inside this chunk
  // Every global load here is independent of the others, so all are issued before
  // the one barrier: the ids of the first batch, this chunk's expert bases, and the
  // whole piece table up to its workspace bound (entries past the plan's count are
  // never read).
  int vv[kAssignBatch];
#pragma unroll
  for (int j = 0; j < kAssignBatch; ++j) {
    const int64_t u = u0 + int64_t(j) * 64 + lane;
    vv[j] = u < u1 ? topk[u] : 0;
  }
  if (have) {
    const int32_t* pp = part + int64_t(c / part_chunks) * E;
    for (int e = lane; e < E; e += 64) run[e] = base[int64_t(c) * E + e] + pp[e];
  }
  for (int i = threadIdx.x; i <= E; i += blockDim.x) s_ptr[i] = piece_ptr[i];
  for (int i = threadIdx.x; i < max_pieces; i += blockDim.x) {
    s_tlo[i] = piece_tlo[i];
    s_base[i] = piece_base[i];
  }
  const bool valid = flags[kFlagPlanValid] != 0;
  __syncthreads();
  if (!have) return;  // whole wavefront leaves; no block barrier follows
  if (!valid) {
    for (int64_t u = u0 + lane; u < u1; u += 64) {
      slot_map[u] = -1;
      src_index[u] = -1;
    }
    return;
  }

  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  for (int s0 = 0; s0 < nsteps; s0 += kAssignBatch) {
    if (s0 > 0) {
#pragma unroll
      for (int j = 0; j < kAssignBatch; ++j) {
        const int64_t u = u0 + int64_t(s0 + j) * 64 + lane;
        vv[j] = u < u1 ? topk[u] : 0;
      }
    }
#pragma unroll
    for (int j = 0; j < kAssignBatch; ++j) {
      if (s0 + j < nsteps) {
        const int64_t u = u0 + int64_t(s0 + j) * 64 + lane;
        const bool act = u < u1;
        const int v = vv[j];
        // lanes holding the same expert id: intersect the ballots of every id bit
        uint64_t m = __ballot(act);
        for (int b = 0; b < nbits; ++b) {
          const bool bit = (v >> b) & 1;
          const uint64_t bal = __ballot(act && bit);
          m &= bit ? bal : ~bal;
        }
        int old = 0;
        const uint64_t below = m & lt_mask;
        if (act && below == 0) old = atomicAdd(&run[v], __popcll(m));  // group leader
        const int leader = act ? __ffsll((unsigned long long)m) - 1 : lane;
        const int grp_base = __shfl(old, leader, 64);
        if (act) {
          const int t = grp_base + __popcll(below);
          int p = s_ptr[v];
          const int p1 = s_ptr[v + 1];
          while (p + 1 < p1 && s_tlo[p + 1] <= t) ++p;
          const int dest = p < p1 ? s_base[p] + t : -1;
          slot_map[u] = dest;
          if (dest >= 0 && int64_t(dest) < NK) src_index[dest] = int32_t(u);
        }
      }
    }
  }
}

}  // namespace moonep

using namespace moonep;

extern "C" int moonep_plan(const moonep_shape* shape, const int32_t* topk_idx, int32_t* cu_seqlens,
                           int32_t* replica_expert, int32_t* slot_map, int32_t* src_index, void* ws,
                           size_t ws_bytes, void* stream) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  const int64_t NK = int64_t(s.R) * s.S * s.K;
  // arrays with no element to touch (an empty layer) may be NULL
  if (!aligned16(cu_seqlens) || !aligned16(ws)) return MOONEP_EINVAL;
  if (NK > 0 && (!aligned16(topk_idx) || !aligned16(slot_map) || !aligned16(src_index)))
    return MOONEP_EINVAL;
  if (s.B > 0 && !aligned16(replica_expert)) return MOONEP_EINVAL;
  const WsLayout w = ws_layout(s);
  if (ws_bytes < w.total) return MOONEP_EWORKSPACE;
  hipStream_t strm = as_stream(stream);
  const int N = s.R * s.S;
  const int nchunk = int(w.nchunk);
  int32_t* flags = ws_ptr<int32_t>(ws, w.flags);
  int32_t* part = ws_ptr<int32_t>(ws, w.part);
  int32_t* counts = ws_ptr<int32_t>(ws, w.counts);
  int32_t* pptr = ws_ptr<int32_t>(ws, w.piece_ptr);
  int32_t* ptlo = ws_ptr<int32_t>(ws, w.piece_tlo);
  int32_t* pbase = ws_ptr<int32_t>(ws, w.piece_base);
  const size_t chunk_lds = size_t(kWavesPerBlock) * s.E * 4;
  const int chunk_blocks = (nchunk + kWavesPerBlock - 1) / kWavesPerBlock;
  const size_t solve_lds = size_t(SolveLds(s.R, s.E, s.B).total) * 4;
  if (solve_lds > 64 * 1024) return MOONEP_ELIMIT;
  // one launch for count, scan and solve when the layer is small and the histograms of
  // a workgroup's chunks fit the same LDS area
  const size_t hist_lds = size_t(kFusedChunks) * s.E * 4;
  const size_t fused_lds = hist_lds > solve_lds ? hist_lds : solve_lds;
  const bool fused = w.nfused > 0 && fused_lds <= 60 * 1024;

  SolveArgs a;
  a.R = s.R; a.S = s.S; a.E = s.E; a.K = s.K; a.B = s.B; a.G = s.E / s.R; a.SK = s.S * s.K;
  a.NK = int64_t(N) * s.K;
  a.part = part; a.npart = int(fused ? w.nfused : w.npart); a.cu = cu_seqlens;
  a.replica = replica_expert; a.piece_ptr = pptr; a.piece_tlo = ptlo; a.piece_base = pbase;
  a.flags = flags;
  if (fused) {
    plan_count_solve_kernel<<<unsigned(w.nfused), kSolveThreads, fused_lds, strm>>>(
        topk_idx, N, nchunk, counts, a);
    if (launch_status()) return MOONEP_EHIP;
  } else {
    if (nchunk > 0) {
      plan_count_kernel<<<chunk_blocks, 256, chunk_lds, strm>>>(topk_idx, N, s.K, s.E, nchunk,
                                                                counts, flags);
      if (launch_status()) return MOONEP_EHIP;
      plan_scan_kernel<<<dim3((s.E + 63) / 64, unsigned(w.npart)), 1024, 0, strm>>>(
          counts, nchunk, s.E, part);
      if (launch_status()) return MOONEP_EHIP;
    }
    plan_solve_kernel<<<1, kSolveThreads, solve_lds, strm>>>(a);
    if (launch_status()) return MOONEP_EHIP;
  }

  if (nchunk > 0) {
    int nbits = 0;
    while ((1 << nbits) < s.E) ++nbits;
    const size_t assign_lds = chunk_lds + (size_t(s.E) + 1 + 2 * size_t(w.max_pieces)) * 4;
    plan_assign_kernel<<<chunk_blocks, 256, assign_lds, strm>>>(
        topk_idx, N, s.K, s.E, nchunk, nbits, counts, part, fused ? kFusedChunks : kScanPart,
        pptr, ptlo, pbase, int(w.max_pieces), flags, slot_map, src_index);
    if (launch_status()) return MOONEP_EHIP;
  }
  return MOONEP_OK;
}
