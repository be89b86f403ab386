// Grouped GEMM over the [E+B, H, H'] expert view on gfx950.
//
// Experts are addressed purely by row index and the active rows come only from
// cu_seqlens, which never leaves the device [ai-maestro.online "Moonshot AI
// open-sources MoonEP", section "The memory contract"]. Launches per call:
//
//   tiles   one workgroup turns cu_seqlens [R, E+B+1] into compact lists of work
//           entries (segment start row, weight row, M offset, length): 256-row
//           M-tiles, and (DGRAD, the fused gate/up projection) a second list of
//           segment tails of at most 128 rows; WGRAD's entries are whole segments,
//           longest first.
//   gemm    a persistent kernel walks entry x N-tile (x M-tile for WGRAD) with
//           256 x 256 tiles; the 32 concurrent tiles of one XCD form a block of 4
//           entries x 8 N-tiles, so they share operand slices in that XCD's L2 (FWD
//           calls of at most 8 N-tiles: blocks of 8 x 4, which the workgroups of each
//           XCD claim in order from a counter of their own).
//   tails   (DGRAD, fused gate/up) the same kernel with 128 x 512 tiles over the
//           tail list: half the MFMAs a 256 x 256 tile spends on a tail of 1..128
//           rows. A plain FWD keeps its tails in the 256 x 256 launch, where the
//           wavefronts of the tile's empty row group sit them out.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 with float32 accumulation (a 128 x 64
// wavefront tile as 8 x 4 blocks: per flop, half the accumulator register traffic
// of the 32 x 32 x 16 form); operands go
// global -> LDS by DMA into a ring of k-steps; operands stored with M or N
// contiguous (the weight in FWD, both operands in WGRAD) stay untransposed in
// LDS and are read with the gfx950 transposing LDS read. A k-step is 64 deep, so
// every DMA of a k-contiguous operand moves whole 128-byte lines. Each wavefront
// holds the fragments of half a step in registers and refills them right behind
// its MFMAs (LDS reads spread between the MFMAs); the one barrier per step
// sits after the last reads of the step's stage, so a two-stage ring keeps the
// DMAs one step ahead and the MFMA pipe never drains at the barrier.
// fp32 path: one thread per output element, each dot product accumulated with error
// compensation (as if in twice the working precision; tiny layers only).
//
// The gate/up projection of the expert FFN can run with its SwiGLU fused into the
// epilogue: with gate and up columns interleaved in 32-column blocks, each 64-column
// group of a wavefront holds the gate and the up value of the same 32 intermediate
// columns, so each lane forms silu(gate) * up from its own accumulators and the
// float32 pre-activation never reaches memory.
#include <atomic>
#include <type_traits>

#include "common.h"

namespace moonep {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;

struct TileEntry {
  int32_t rowbase;  // global buffer row of the segment's first slot: q*SK + cu[q][i]
  int32_t wrow;     // W_all row (FWD/DGRAD) / grad row (WGRAD: < E grad_home, else reduce_buf+E)
  int32_t m0;       // first segment row of this entry (FWD/DGRAD), 0 for WGRAD
  int32_t n;        // segment length
};

// ------------------------------------------------------------------ tile list
__device__ inline int wave_scan_incl(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Whole-segment entries (WGRAD) are listed longest first when there are at most
// this many: the length of a WGRAD tile's k-loop is its segment's, which ranges
// over orders of magnitude under skew, and the persistent grid takes tiles in list
// order, so long tiles at the end leave most CUs idle. A training plan has at most
// E + R*B = 2E <= 2048 non-empty segments, so every planned WGRAD is sorted; larger
// counts (cu_seqlens from elsewhere, up to R*(E+B) <= 8192 rows) keep plan order.
constexpr int kSortMax = 4096;
// Entries of a list that the tile-list kernel builds in LDS (64 KiB); longer lists are
// built in place in memory.
constexpr int kStageMax = 4096;
static_assert(kSortMax * sizeof(uint64_t) <= kStageMax * 16, "sort keys share the LDS list buffer");

// M-tiles of bm rows per segment (bm = 0: one entry per whole segment). With
// tail > 0 a segment's last M-tile goes to a second list when it has at most
// `tail` rows: those are computed by a kernel with tail-row M-tiles and twice
// the N width, so a short tail costs half as many MFMAs. With bm = 0 and
// longest_first the entries are ordered by segment length, descending (ties in
// (rank, row) order). With group > 0, each run of `group` consecutive entries lists its
// entries of at most bm/2 rows last (see below). Every tile owns its outputs, so no
// order changes a result.
__global__ __launch_bounds__(1024) void gemm_tiles_kernel(const int32_t* __restrict__ cu, int R,
                                                          int E, int B, int SK, int bm, int tail,
                                                          bool longest_first,
                                                          TileEntry* __restrict__ tiles,
                                                          int32_t* __restrict__ ntiles,
                                                          int max_tiles,
                                                          TileEntry* __restrict__ tails,
                                                          int32_t* __restrict__ ntails,
                                                          int max_tails,
                                                          int32_t* __restrict__ qcnt, int group) {
  // the tile-queue counters of the GEMM launches that follow (full tiles, then tails)
  if (qcnt && threadIdx.x < 2 * kQueueWords) qcnt[threadIdx.x] = 0;
  __shared__ int swave[2][17];
  // sort keys (WGRAD) or the staged list (every other call): one buffer, two uses
  __shared__ __align__(16) char s_buf[kStageMax * sizeof(TileEntry)];
  uint64_t* skey = reinterpret_cast<uint64_t*>(s_buf);
  TileEntry* s_ent = reinterpret_cast<TileEntry*>(s_buf);
  const int EB = E + B, total = R * EB;
  const int per = (total + 1023) / 1024;
  const int i0 = threadIdx.x * per, i1 = min(total, i0 + per);
  // full tiles of a segment of n rows, and whether its tail goes to the second list
  auto split = [&](int n, int& nfull, int& ntail) {
    if (bm <= 0) { nfull = 1; ntail = 0; return; }
    nfull = (n + bm - 1) / bm;
    const int rem = n - (nfull - 1) * bm;
    ntail = (tail > 0 && rem <= tail) ? 1 : 0;
    nfull -= ntail;
  };
  int cnt = 0, cnt_tail = 0;
  for (int idx = i0; idx < i1; ++idx) {
    const int q = idx / EB, i = idx % EB;
    const int n = cu[q * (EB + 1) + i + 1] - cu[q * (EB + 1) + i];
    if (n <= 0) continue;
    int f, t;
    split(n, f, t);
    cnt += f;
    cnt_tail += t;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_scan_incl(cnt);
  const int incl_t = wave_scan_incl(cnt_tail);
  if (lane == 63) {
    swave[0][w] = incl;
    swave[1][w] = incl_t;
  }
  __syncthreads();
  if (w < 2) {
    const int x = lane < 16 ? swave[w][lane] : 0;
    const int xi = wave_scan_incl(x);
    if (lane < 16) swave[w][lane] = xi - x;
    if (lane == 15) swave[w][16] = xi;
  }
  __syncthreads();
  int k = swave[0][w] + incl - cnt;
  int kt = swave[1][w] + incl_t - cnt_tail;
  const int count = swave[0][16];
  if (threadIdx.x == 0) {
    *ntiles = min(count, max_tiles);
    *ntails = min(swave[1][16], max_tails);
  }
  if (bm <= 0 && longest_first && count <= kSortMax && count <= max_tiles) {
    // key: (length descending, segment index ascending); padding sorts last
    for (int idx = i0; idx < i1; ++idx) {
      const int q = idx / EB, i = idx % EB;
      const int n = cu[q * (EB + 1) + i + 1] - cu[q * (EB + 1) + i];
      if (n <= 0) continue;
      skey[k++] = (uint64_t(0x7FFFFFFF - n) << 32) | uint32_t(idx);
    }
    int P = 1;
    while (P < count) P <<= 1;
    for (int j = count + threadIdx.x; j < P; j += 1024) skey[j] = ~uint64_t(0);
    __syncthreads();
    // bitonic sort of skey[0, P), ascending
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = threadIdx.x; t < P / 2; t += 1024) {
          const int lo = 2 * stride * (t / stride) + t % stride, hi = lo + stride;
          const uint64_t a = skey[lo], b = skey[hi];
          if ((a > b) == ((lo & size) == 0)) {
            skey[lo] = b;
            skey[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    for (int j = threadIdx.x; j < count; j += 1024) {
      const int idx = int(uint32_t(skey[j]));
      const int q = idx / EB, i = idx % EB;
      const int c0 = cu[q * (EB + 1) + i];
      const int n = cu[q * (EB + 1) + i + 1] - c0;
      tiles[j] = TileEntry{q * SK + c0, i < E ? i : E + q * B + (i - E), 0, n};
    }
    return;
  }
  // A list that fits is built in LDS, reordered there and copied out in one coalesced
  // pass, instead of being written to memory and read back: at 524288 slots, H = 7168,
  // H' = 2048 (about 2250 entries) the kernel's chain of memory round trips took 24-33 us,
  // against 12-17 us this way.
  const int listed = min(count, max_tiles);
  const bool staged = listed <= kStageMax;   // uniform
  TileEntry* out = staged ? s_ent : tiles;
  for (int idx = i0; idx < i1; ++idx) {
    const int q = idx / EB, i = idx % EB;
    const int c0 = cu[q * (EB + 1) + i];
    const int n = cu[q * (EB + 1) + i + 1] - c0;
    if (n <= 0) continue;
    const int wrow = i < E ? i : E + q * B + (i - E);
    int f, t;
    split(n, f, t);
    const int step = bm > 0 ? bm : n;
    for (int j = 0; j < f; ++j) {
      if (k < listed) out[k] = TileEntry{q * SK + c0, wrow, j * step, n};
      ++k;
    }
    if (t) {
      if (kt < max_tails) tails[kt] = TileEntry{q * SK + c0, wrow, f * step, n};
      ++kt;
    }
  }
  // A segment's last tile of at most bm/2 rows takes about half a tile's time (its second
  // row group idles). The workgroups of an XCD claim its tiles first come first served,
  // and its tiles share operand lines in L2 only while they stay within a few steps of
  // each other. Listing such entries last in each run of `group` entries (one tile-order
  // block, one round of the XCD's queue) hands the short tiles to the workgroups that
  // finished the previous round last, so the XCD's workgroups converge instead of drifting
  // apart. A/B, bit-identical: FWD at H = 7168, H' = 2048 -0.9 to -2.2% at four imbalance
  // points, its fetch 63.4 -> 53.8 GB per call; within noise at H' = 1536 and 1408.
  if (group > 0 && group <= 8) {
    __syncthreads();   // the list is written
    for (int base = threadIdx.x * group; base < listed; base += 1024 * group) {
      // unrolled, so that e[] stays in registers
      TileEntry e[8];
      const int m = min(group, listed - base);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < m) e[i] = out[base + i];
      int o = base;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < m && e[i].n - e[i].m0 > bm / 2) out[o++] = e[i];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < m && e[i].n - e[i].m0 <= bm / 2) out[o++] = e[i];
    }
  }
  if (staged) {
    __syncthreads();   // the list is complete in LDS
    for (int j = threadIdx.x; j < listed; j += 1024) tiles[j] = s_ent[j];
  }
}

// ------------------------------------------------------------------ staging
// Operands move global -> LDS by direct DMA (buffer_load_dwordx4 ... lds: lane l
// of a wavefront writes 16 bytes at M0 + 16*l), through buffer resources: a
// descriptor (base, byte range) in scalar registers plus a 32-bit offset per
// lane; loads past the range return 0, stores past it are dropped. Partial
// tiles therefore need no branches. No operand passes through registers, so
// the k-loop keeps several steps in flight in a ring of LDS stages.
//
// LDS layouts of one 64-deep k-step (16-byte chunks XOR-swizzled so that the
// fragment reads of 8 or 16 lanes at a time hit distinct banks):
//   k-contiguous operand   [ROWS][64]: 128-byte rows, chunk c of row r at c ^ swz_k(r).
//     One DMA instruction moves 8 whole rows, each a full 128-byte line: 32-deep
//     steps (64-byte half lines) measured 4% slower at the bench shape.
//   m/n-contiguous operand [64][COLS]: one row per k, chunk c of row k at c ^ swz_mn(k);
//     read with ds_read_b64_tr_b16, which hands each lane 4 consecutive k of one
//     column, the MFMA operand layout, without a transpose anywhere else.
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcFlags = 0x00020000;      // raw (unswizzled) 32-bit data, gfx9 family
constexpr uint32_t kOffNone = 0x80000000u;  // an offset past every range used here
constexpr int kBK = 64;                     // k per pipeline step
constexpr int kBlockE = 4, kBlockN = 8;     // FWD/DGRAD tile order block
constexpr int kTailGroup = 8;               // entries per tile-order block of queued FWD calls
static_assert(kTailGroup <= 8, "the tile-list kernel reorders groups of at most 8 entries");
constexpr int kEpiAhead = 4;                // WGRAD epilogue: row blocks read ahead of the stores
// Cache policy of streaming output stores (nt sc1), and the longest reduction for which
// DGRAD stores its float32 output that way. With 22 k-steps per tile (H' = 1408) the
// output leaves fast enough to push operand lines out of L2: streaming stores made that
// DGRAD 4.3% faster (2970-3003 -> 2848-2868 us, three A/B pairs on one box), while they
// were neutral or slightly slower for every longer reduction and for FWD (the FFN down
// projection 1% slower).
constexpr int kStreamStore = 18;
constexpr int kStreamOutMaxK = 1536;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // the range is uniform; readfirstlane keeps it (and the descriptor) in scalar
  // registers even where it was computed with 64-bit vector compares
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kRsrcFlags);
}

__device__ inline uint32_t clamp_bytes(int64_t b) {
  return b <= 0 ? 0u : (b >= int64_t(kOffNone) ? kOffNone : uint32_t(b));
}

// One 16-byte-per-lane DMA into LDS at byte address lds (uniform). Issued as
// inline assembly so that the compiler's wait-count pass does not wait for all
// outstanding DMAs at every LDS read; the k-loop waits for exactly the steps it
// needs (wait_vm).
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Wait until at most n of this wavefront's vector memory operations are pending.
template <int n>
__device__ inline void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // s_waitcnt simm16: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and
  // lgkmcnt left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ inline int swz_k(int r) { return (r >> 1) & 7; }
// the 4 k-rows one 16-lane group reads take disjoint 32-byte column slots of a
// 256-byte bank window (k & 3), and the group 8 rows further on, which shares the
// half-wavefront's pass, takes the 8 slots left free (k & 8)
__device__ inline int swz_mn(int k) {
  return ((k & 1) ? 6 : 0) ^ ((k & 2) ? 10 : 0) ^ ((k & 8) ? 2 : 0);
}

typedef __attribute__((address_space(3))) char lds_char;

// LDS byte address of a pointer into __shared__ memory (address-space cast).
__device__ inline uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_char*)p));
}

// k-contiguous operand tile: ROWS rows x 64 k.
template <int ROWS, int NWAVES>
struct OpK {
  static constexpr int ROWB = kBK * 2;
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int READS = 1;               // LDS reads per MFMA operand
  static constexpr int INSTR = BYTES / 1024;  // 8 rows per wavefront DMA
  static constexpr int PER_WAVE = INSTR / NWAVES;
  static_assert(INSTR % NWAVES == 0, "DMA split");
  // rsrc base at (row 0, k0); ld in bytes; rows past the range read 0
  __device__ static inline void issue(__amdgpu_buffer_rsrc_t rs, uint32_t ld, uint32_t lds,
                                      int wave, int lane, int /*cols_valid*/) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int b = wave + i * NWAVES;
      const int row = b * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz_k(row);
      dma16(rs, uint32_t(row) * ld + c * 16, lds + b * 1024);
    }
  }
  // MFMA operand: row rbase + lane%16, k = 32*ks + 8*(lane/16) .. +8
  __device__ static inline bf16x8_t frag(const char* st, int rbase, int ks, int lane) {
    const int row = rbase + (lane & 15);
    const int c = ks * 4 + (lane >> 4);
    return *reinterpret_cast<const bf16x8_t*>(st + row * ROWB + ((c ^ swz_k(row)) << 4));
  }
};

// m/n-contiguous operand tile: 64 k-rows x COLS.
template <int COLS, int NWAVES>
struct OpMN {
  static constexpr int ROWB = COLS * 2;
  static constexpr int CPR = ROWB / 16;         // chunks per row
  static constexpr int READS = 2;               // LDS reads per MFMA operand
  static constexpr int BYTES = kBK * ROWB;
  static constexpr int INSTR = BYTES / 1024;
  static constexpr int RPI = 1024 / ROWB;       // k rows per wavefront DMA
  static constexpr int PER_WAVE = INSTR / NWAVES;
  static_assert(INSTR % NWAVES == 0 && RPI >= 1, "DMA split");
  // rsrc base at (k0, col 0); ld in bytes; k rows past the range and columns at or
  // past cols_valid read 0
  __device__ static inline void issue(__amdgpu_buffer_rsrc_t rs, uint32_t ld, uint32_t lds,
                                      int wave, int lane, int cols_valid) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int b = wave + i * NWAVES;
      const int k = b * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz_mn(k);
      const uint32_t off = c * 8 < cols_valid ? uint32_t(k) * ld + c * 16 : kOffNone;
      dma16(rs, off, lds + b * 1024);
    }
  }
  // MFMA operand: column cbase + lane%16, k = 32*ks + 8*(lane/16) .. +8, as two
  // transposed 4x16 reads per 16-lane group: lane i of the group addresses k-row i/4
  // and columns 4*(i%4) .. +4 and receives the 4 k of column i
  __device__ static inline bf16x8_t frag(const char* st, int cbase, int ks, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int col = cbase + 4 * (i & 3);
    const int c = col >> 3, half = (col >> 2) & 1;
    const int k0 = ks * 32 + g * 8 + (i >> 2);
    v4s_t v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + 4 * h;
      const char* p = st + k * ROWB + ((c ^ swz_mn(k)) << 4) + half * 8;
      v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s_t*)((const lds_char*)p));
    }
    const v4i_t w = {int((uint16_t)v[0][0] | ((uint32_t)(uint16_t)v[0][1] << 16)),
                     int((uint16_t)v[0][2] | ((uint32_t)(uint16_t)v[0][3] << 16)),
                     int((uint16_t)v[1][0] | ((uint32_t)(uint16_t)v[1][1] << 16)),
                     int((uint16_t)v[1][2] | ((uint32_t)(uint16_t)v[1][3] << 16))};
    return __builtin_bit_cast(bf16x8_t, w);
  }
};

// ------------------------------------------------------------------ bf16 kernel
struct GemmArgs {
  const uint16_t* a;
  const uint16_t* b;
  float* c;
  float* grad_home;
  float* reduce_buf;
  const TileEntry* tiles;
  const int32_t* ntiles;
  int H, Hp, E;
  uint16_t* act;      // SwiGLU epilogue: bf16 [rows, Hp/2]
  uint16_t* h_saved;  // SwiGLU epilogue: NULL or bf16 [rows, Hp]
  int32_t* qcnt;      // 8 per-XCD tile-queue counters, zero at launch (NULL: static order)
};

template <int OP, int BM, int BN, int WAVES_M, int WAVES_N, bool SWIGLU = false,
          bool STREAM_OUT = false, int STAGES = 2, bool HALFN = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 16, FN = WN / 16;   // 16 x 16 MFMA blocks per wavefront
  // WGRAD multiplies with the operands swapped, so each accumulator block is the
  // transpose and a lane holds 4 consecutive columns of one row: its += epilogue
  // moves 16 bytes per load and store (a quarter of the instructions; 5% faster at
  // H = 4096, H' = 1408). FWD and DGRAD keep the direct form, which measured faster
  // for their plain stores.
  constexpr bool SWAP = OP == MOONEP_WGRAD;
  static_assert(FM >= 1 && FN >= 1, "tile shape");
  static_assert(!SWIGLU || (OP == MOONEP_FWD && FN % 4 == 0 && kSwigluBlock == 32),
                "SwiGLU epilogue: a wavefront holds whole (gate, up) 32-column block pairs");
  // A stored k-contiguous except in WGRAD; B stored n-contiguous except in DGRAD
  // Wavefronts that issue the DMAs. The two wavefronts on each SIMD (w and w + NW/2)
  // share its matrix pipe unevenly: with every wavefront issuing an equal share, the
  // older one reaches each barrier early and waits there about a third of the step
  // (s_memtime probe), and the other is on the critical path. In FWD and WGRAD the
  // older ones (w < NW/2) issue every DMA, twice their share, and the others issue none
  // and never wait on the vector-memory counter; the barrier still follows every
  // issuing wavefront's wait for its own share. Bit-identical. A/B on one box: FWD at
  // H = 7168, H' = 2048 13.54 -> 13.17 ms, at H = 4096, H' = 1536 -3 to -4%, WGRAD at
  // H = 4096, H' = 1408 -4%; DGRAD measured no change and keeps all wavefronts. Issue
  // counts in between (one operand from w < NW/2, the other from all: 12 and 4 per step)
  // were 6-10% slower than the equal split, so what pays is wavefronts free of DMA waits.
  // The 128 x 512 tail tiles (one row group) keep every wavefront issuing: 0.2-0.5%
  // faster there than the split.
  constexpr int DW = WAVES_M != 2 || OP == MOONEP_DGRAD ? NW : NW / 2;
  using OA = typename std::conditional<OP == MOONEP_WGRAD, OpMN<BM, DW>, OpK<BM, DW>>::type;
  using OB = typename std::conditional<OP == MOONEP_DGRAD, OpK<BN, DW>, OpMN<BN, DW>>::type;
  constexpr int DMA_PER_STEP = OA::PER_WAVE + OB::PER_WAVE;   // per issuing wavefront
  constexpr int STAGE = OA::BYTES + OB::BYTES;
  static_assert(STAGES >= 2, "LDS ring depth");
  __shared__ __align__(1024) char smem[STAGES * STAGE];

  const int Ndim = OP == MOONEP_DGRAD ? g.H : g.Hp;   // columns of C
  const int Kfix = OP == MOONEP_FWD ? g.H : g.Hp;     // FWD/DGRAD reduction length
  const int NT = (Ndim + BN - 1) / BN;
  const int MT = OP == MOONEP_WGRAD ? (g.H + BM - 1) / BM : 1;
  const int64_t nent = *g.ntiles;
  const int64_t total = nent * MT * NT;
  const int64_t wsz = int64_t(g.H) * g.Hp;
  const uint32_t lda_b = uint32_t(OP == MOONEP_DGRAD ? g.Hp : g.H) * 2;   // bytes per A row
  const uint32_t ldb_b = uint32_t(g.Hp) * 2;                              // bytes per B row

  // the wavefront id is uniform: keep it (and every LDS address derived from it)
  // in scalar registers
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const uint32_t lds0 = lds_addr(smem);

  // XCD-aware order: the workgroups of one XCD take a contiguous run of tiles.
  const int G = gridDim.x;
  const int slot = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;

  // Per-XCD tile queues (FWD on 256 x 256 tiles, at most 8 N-tiles): the workgroups of
  // XCD x take its tiles of the static order, (q / P) * G + x * P + q % P for queue
  // position q, first come first served, so the tiles in flight on an XCD stay one
  // contiguous window however far its workgroups drift apart. Thread 0 claims the next
  // tile during the current one. A/B, bit-identical: FWD at H = 7168, H' = 2048 -0.5%
  // (HBM reads 52.9 -> 48.1 GB per call), at H = 4096, H' = 1408 -1.5%. Wider outputs
  // measured slower (the fused gate/up + SwiGLU, 16 N-tiles, +3.5%; H' -> H = 7168, 28
  // N-tiles, +0.5%), as did DGRAD (+0.8%) and the 128 x 128 tiles of small calls (+4%, a
  // claim per short tile); they keep the static order, as do WGRAD (which prefetches its
  // next tile's first step) and the 128 x 512 tail tiles (whose ring fills the LDS).
  constexpr bool DYN = OP == MOONEP_FWD && !SWIGLU && BM == 256 && BN == 256;
  const bool dyn = DYN && g.qcnt != nullptr && G % 8 == 0 && NT <= 8;
  // the tile of task tau: its entry, first row and column, valid rows and columns,
  // and reduction length
  struct Task {
    TileEntry te;
    int m0, n0, rows_valid, cols_valid, kdim;
  };
  auto task_at = [&](int64_t tau) {
    int64_t ent;
    int mt, nt;
    if (OP == MOONEP_WGRAD) {
      ent = tau / (int64_t(MT) * NT);
      const int rem = int(tau % (int64_t(MT) * NT));
      mt = rem / NT;
      nt = rem % NT;
    } else {
      // blocks of kBlockE entries x kBlockN N-tiles, so that the 32 concurrent tiles of
      // an XCD reuse each weight N-tile for four M-tiles and each activation tile for
      // eight N-tiles. With the tile queues, whose tiles in flight stay together, blocks
      // of 8 x 4 measured 0.8% faster at H = 7168, H' = 2048 (each weight N-tile serves
      // eight M-tiles, each activation tile is read twice).
      const int bE = dyn ? 8 : kBlockE, bN = dyn ? 4 : kBlockN;
      const int64_t eb = tau / (int64_t(bE) * NT);
      const int j = int(tau % (int64_t(bE) * NT));
      const int ge = int(min(int64_t(bE), nent - eb * bE));
      const int nb = j / (ge * bN), jj = j % (ge * bN);
      const int wb = min(bN, NT - nb * bN);
      ent = eb * bE + jj / wb;
      mt = 0;
      nt = nb * bN + jj % wb;
    }
    Task t;
    // the entry is uniform; readfirstlane keeps it (and the buffer descriptors built
    // from it) in scalar registers wherever it is loaded
    const TileEntry e = g.tiles[ent];
    t.te = TileEntry{__builtin_amdgcn_readfirstlane(e.rowbase), __builtin_amdgcn_readfirstlane(e.wrow),
                     __builtin_amdgcn_readfirstlane(e.m0), __builtin_amdgcn_readfirstlane(e.n)};
    t.n0 = nt * BN;
    t.cols_valid = min(BN, Ndim - t.n0);
    if (OP == MOONEP_WGRAD) {
      t.m0 = mt * BM;
      t.rows_valid = min(BM, g.H - t.m0);
      t.kdim = t.te.n;
    } else {
      t.m0 = t.te.m0;
      t.rows_valid = min(BM, t.te.n - t.te.m0);
      t.kdim = Kfix;
    }
    return t;
  };
  // issue the DMAs of k-step kt of task t into the ring stage at LDS address st
  auto issue_task = [&](const Task& t, int kt, uint32_t st) {
    if (wid >= DW) return;   // uniform per wavefront
    const int k0 = kt * kBK;
    const TileEntry& te = t.te;
    const int m0 = t.m0, n0 = t.n0, rows_valid = t.rows_valid, cols_valid = t.cols_valid;
    const int kdim = t.kdim;
    if constexpr (OP == MOONEP_FWD) {
      OA::issue(make_rsrc(g.a + (int64_t(te.rowbase) + m0) * g.H + k0,
                          clamp_bytes(int64_t(rows_valid) * lda_b)), lda_b, st, wid, lane, 0);
      OB::issue(make_rsrc(g.b + int64_t(te.wrow) * wsz + int64_t(k0) * g.Hp + n0,
                          clamp_bytes(int64_t(kdim - k0) * ldb_b)), ldb_b, st + OA::BYTES,
                wid, lane, cols_valid);
    } else if constexpr (OP == MOONEP_DGRAD) {
      OA::issue(make_rsrc(g.a + (int64_t(te.rowbase) + m0) * g.Hp + k0,
                          clamp_bytes(int64_t(rows_valid) * lda_b)), lda_b, st, wid, lane, 0);
      OB::issue(make_rsrc(g.b + int64_t(te.wrow) * wsz + int64_t(n0) * g.Hp + k0,
                          clamp_bytes(int64_t(cols_valid) * ldb_b)), ldb_b, st + OA::BYTES,
                wid, lane, 0);
    } else {
      OA::issue(make_rsrc(g.a + (int64_t(te.rowbase) + k0) * g.H + m0,
                          clamp_bytes(int64_t(kdim - k0) * lda_b)), lda_b, st, wid, lane,
                rows_valid);
      OB::issue(make_rsrc(g.b + (int64_t(te.rowbase) + k0) * g.Hp + n0,
                          clamp_bytes(int64_t(kdim - k0) * ldb_b)), ldb_b, st + OA::BYTES,
                wid, lane, cols_valid);
    }
  };

  // Ring stage of k-step kt is (base + kt) % 2. In WGRAD the last step of a tile
  // issues the next tile's step 0 into the stage its own reads have just released
  // (its barrier orders every wavefront's reads of it before the DMA), so that DMA
  // runs under the last half step and the += epilogue; the next tile's base is that
  // stage. WGRAD measured 3.5% faster at H = 4096, H' = 1408; FWD within noise and
  // DGRAD (22 k-steps per tile there) 2% slower, so they start every tile afresh.
  constexpr bool NEXT_STEP0 = OP == MOONEP_WGRAD && STAGES == 2;
  int base = 0;
  bool step0_issued = false;
  const int xcd = int(blockIdx.x % 8), per_xcd = G / 8;
  __shared__ int s_claim[1];   // referenced only when DYN (otherwise not allocated)
  auto claim = [&]() {
    if constexpr (DYN) {
      const int q = atomicAdd(g.qcnt + xcd, 1);
      s_claim[0] = (q / per_xcd) * G + xcd * per_xcd + q % per_xcd;
    }
  };
  auto claimed = [&]() -> int64_t {
    if constexpr (DYN) return __builtin_amdgcn_readfirstlane(s_claim[0]);
    else return 0;
  };
  int64_t tau = slot;
  if (dyn) {
    if (threadIdx.x == 0) claim();
    __syncthreads();
    tau = claimed();
  }
  for (; tau < total; tau = dyn ? claimed() : tau + G) {
    const Task cur = task_at(tau);
    const TileEntry te = cur.te;
    const int m0 = cur.m0, n0 = cur.n0, rows_valid = cur.rows_valid;
    const int cols_valid = cur.cols_valid, kdim = cur.kdim;
    const int kiters = (kdim + kBK - 1) / kBK;
    const bool has_next = NEXT_STEP0 && tau + G < total;
    auto stage = [&](int kt) {
      if constexpr ((STAGES & (STAGES - 1)) == 0) return uint32_t((base + kt) & (STAGES - 1)) * STAGE;
      else return uint32_t(unsigned(base + kt) % STAGES) * STAGE;
    };
    auto issue = [&](int kt) { issue_task(cur, kt, lds0 + stage(kt)); };
    // wait until at most n later steps of this wavefront's DMAs are in flight
    auto wait_steps = [&](int n) {
      if (wid >= DW) return;   // no DMAs of its own
      if constexpr (STAGES > 3) {
        if (n >= 3) { wait_vm<3 * DMA_PER_STEP>(); return; }
      }
      if constexpr (STAGES > 2) {
        if (n == 2) { wait_vm<2 * DMA_PER_STEP>(); return; }
      }
      if (n == 1) wait_vm<DMA_PER_STEP>();
      else wait_vm<0>();
    };

    // the tile's MFMAs, ring and epilogue for a wavefront of FM 16-row fragments whose
    // rows start at row0 and whose WN columns start at col0 of the tile; an idle
    // wavefront (HALFN) only keeps the ring's DMAs and barriers
    auto tile = [&](auto fm_c, int row0, int col0_arg, bool idle) {
      constexpr int FM = decltype(fm_c)::value;
      const int col0 = HALFN ? col0_arg : wn * WN;
      // A tile whose valid rows all lie in the first row group (a segment's last tile)
      // leaves the second group's wavefronts without a row: they skip the MFMAs, LDS
      // reads and stores, issue their share of the DMAs and meet every barrier, so their
      // SIMD partners run alone for about half the tile's time. This is what a plain FWD
      // does with its segment tails of at most 128 rows: run there, next to the same
      // segment's full tiles, each tail finds the weight slice in L2, where the tail
      // launch re-read it from HBM. A/B, bit-identical: FWD at H = 7168, H' = 2048 -0.3
      // to -0.4%, at H = 4096, H' = 1536 -2.2%, at H = 4096, H' = 1408 -3.2%, the FFN down
      // projection (H' -> H = 7168) -2.3%. DGRAD (+1%) and the fused gate/up projection
      // (+6% at one of four imbalance points) measured slower and keep the tail launch.
      if constexpr (HALFN || (OP != MOONEP_WGRAD && WAVES_M == 2)) {
        if ((HALFN && idle) ||
            (OP != MOONEP_WGRAD && WAVES_M == 2 && row0 >= rows_valid)) {   // uniform
          __syncthreads();
          if (!step0_issued) issue(0);
#pragma unroll
          for (int k = 1; k < STAGES; ++k)
            if (k < kiters) issue(k);
          wait_steps(min(STAGES, kiters) - 1);
          __syncthreads();
          for (int kt = 0; kt < kiters; ++kt) {
            const bool more = kt + 1 < kiters;
            if (more) wait_steps(min(kt + STAGES - 1, kiters - 1) - (kt + 1));
            __syncthreads();
            if (kt + STAGES < kiters) issue(kt + STAGES);
            else if (!more && has_next) issue_task(task_at(tau + G), 0, lds0 + stage(kt));
          }
          if constexpr (NEXT_STEP0) {
            step0_issued = has_next;
            base = (base + kiters - 1) & 1;
          }
          return;
        }
      }
      floatx4_t acc[FM][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

      // every wavefront has finished reading the ring (previous tile) before refilling it
      __syncthreads();
      if (!step0_issued) issue(0);
#pragma unroll
      for (int k = 1; k < STAGES; ++k)
        if (k < kiters) issue(k);

      // The fragments of half a step (one 32-deep substep: FM + FN operands of 4
      // registers) live in registers: a whole step's would need 96 registers beside
      // the 128 accumulators and spills. Step kt:
      //   first half   MFMAs of substep 0; its registers refilled with substep 1 of
      //                the same step (the last reads of its stage)
      //   barrier      step kt+1 is visible to every wavefront, and every read of
      //                stage kt % 2 has completed, so step kt+2 is issued into it
      //   second half  MFMAs of substep 1; registers refilled with substep 0 of
      //                step kt+1
      // LDS reads are spread between the MFMAs, so they run under the MFMAs and the
      // MFMA pipe never drains at the barrier.
      constexpr int KS = kBK / 32;
      constexpr int HALF = KS / 2;
      bf16x8_t fa[HALF][FM], fb[HALF][FN];
      auto load = [&](int kt, int ks, int buf) {
        const char* st = smem + stage(kt);
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = OA::frag(st, row0 + i * 16, ks, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = OB::frag(st + OA::BYTES, col0 + j * 16, ks, lane);
      };
      auto mfma = [&](int buf, int i, int j) {
        if constexpr (SWAP)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
      };
      // MFMA order inside a half step. Row-outer order frees each A fragment after its
      // row, but every B fragment only in the last row, so all the B refills are issued at
      // the end and the next half needs them at once. The two wavefronts of a SIMD do not
      // share the matrix pipe evenly: the older one reaches the barrier first and waits
      // there about a third of each step (s_memtime probe), and the other, running alone,
      // stalls on those refills. Two column blocks (every row with the first FN/2 columns,
      // then every row with the rest) free the first block's B fragments for refill under
      // the second block; the second block's are needed only halfway through the next half,
      // and each A fragment only at its row in the next half's first block. Every
      // accumulator keeps its k order, so results are bit-identical. Measured: FWD at
      // H = 7168, H' = 2048 13.70 -> 13.44 ms, at H = 4096, H' = 1408 -2.5%; DGRAD unchanged.
      // WGRAD, whose A refills are transposed reads too, has more refills than the second
      // block has MFMAs and keeps row-outer order (the split spread over its MFMAs measured
      // no gain there).
      constexpr bool SPLIT = FN >= 4 && FN % 2 == 0 &&
                             FM * OA::READS + (FN / 2) * OB::READS <= FM * FN / 2;
      auto mfmas = [&](int buf) {
        if constexpr (SPLIT) {
#pragma unroll
          for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = jb * (FN / 2); j < (jb + 1) * (FN / 2); ++j) mfma(buf, i, j);
        } else {
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) mfma(buf, i, j);
        }
      };
      // LDS reads per substep: one per k-contiguous fragment, two per transposed one
      constexpr int READS = FM * OA::READS + FN * OB::READS;
      constexpr int PER_READ = (FM * FN) / READS > 0 ? (FM * FN) / READS : 1;
      auto interleave = [&]() {
        if constexpr (SPLIT) {
          constexpr int HALFM = FM * FN / 2;
          constexpr int EARLY = FM * OA::READS + (FN / 2) * OB::READS;
          // no refill fits under the first block; under the second, one LDS read after each
          // MFMA for the refills freed so far, and the last block's B refills at the end
          __builtin_amdgcn_sched_group_barrier(0x008, HALFM, 0);      // first column block
#pragma unroll
          for (int q = 0; q < EARLY; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // one LDS read
          }
          if constexpr (HALFM > EARLY)
            __builtin_amdgcn_sched_group_barrier(0x008, HALFM - EARLY, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, READS - EARLY, 0);
        } else {
#pragma unroll
          for (int q = 0; q < READS; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, PER_READ, 0);   // MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // one LDS read
          }
        }
      };
      // step 0 landed (the later steps of the ring may still be in flight)
      wait_steps(min(STAGES, kiters) - 1);
      __syncthreads();
      // the next tile, read after the k-loop's barriers (at least one)
      if (dyn && threadIdx.x == 0) claim();
#pragma unroll
      for (int h = 0; h < HALF; ++h) load(0, h, h);
      for (int kt = 0; kt < kiters; ++kt) {
        const bool more = kt + 1 < kiters;
#pragma unroll
        for (int h = 0; h < HALF; ++h) {
          mfmas(h);
          load(kt, HALF + h, h);
          interleave();
        }
        // this wavefront's DMAs of step kt+1 (steps up to kt+STAGES-1 may be in flight)
        if (more) wait_steps(min(kt + STAGES - 1, kiters - 1) - (kt + 1));
        __syncthreads();
        if (kt + STAGES < kiters) issue(kt + STAGES);
        else if (!more && has_next) issue_task(task_at(tau + G), 0, lds0 + stage(kt));
#pragma unroll
        for (int h = 0; h < HALF; ++h) {
          mfmas(h);
          // after the last step: read a stage with no DMA in flight into it (in bounds,
          // values unused): this step's, or the other one when the next tile's step 0
          // is on its way into this one
          load(more || NEXT_STEP0 ? kt + 1 : kt, h, h);
          interleave();
        }
      }
      if constexpr (NEXT_STEP0) {
        step0_issued = has_next;
        base = (base + kiters - 1) & 1;
      }

      // epilogue: lane holds column lane % 16 and rows 4 * (lane / 16) + r (r = 0..3)
      // of each 16 x 16 block; rows past rows_valid fall outside the range.
      const int r16 = lane & 15;
      const uint32_t lane_rows = uint32_t(row0 + (lane >> 4) * 4);
      if constexpr (SWIGLU) {
        // in each 64-column group jp of the wavefront, blocks 4jp, 4jp+1 hold the gate
        // and blocks 4jp+2, 4jp+3 the up value of intermediate columns
        // n0/2 + col0/2 + jp*32 + (0..31); a partial tile ends on a 64-column boundary,
        // so each group is all in or all out
        const int hact = g.Hp / 2;
        const int64_t row0 = int64_t(te.rowbase) + m0;
        const __amdgpu_buffer_rsrc_t ars =
            make_rsrc(g.act + row0 * hact + n0 / 2, clamp_bytes(int64_t(rows_valid) * hact * 2));
        const uint32_t arow = lane_rows * hact * 2;
        uint32_t la[FN / 4];
#pragma unroll
        for (int jp = 0; jp < FN / 4; ++jp)
          la[jp] = col0 + jp * 64 < cols_valid
                       ? arow + uint32_t(col0 / 2 + jp * kSwigluBlock + r16) * 2
                       : kOffNone;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t rowoff = uint32_t(i * 16 + r) * hact * 2;
#pragma unroll
            for (int jp = 0; jp < FN / 4; ++jp)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const float v = swiglu_f32(acc[i][4 * jp + h][r], acc[i][4 * jp + 2 + h][r]);
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16_rne_bits(v), ars,
                                                      la[jp] + rowoff + h * 32, 0, 0);
              }
          }
        if (g.h_saved) {
          const __amdgpu_buffer_rsrc_t hrs = make_rsrc(
              g.h_saved + row0 * g.Hp + n0, clamp_bytes(int64_t(rows_valid) * g.Hp * 2));
          const uint32_t hrow = lane_rows * g.Hp * 2;
          uint32_t lh[FN];
#pragma unroll
          for (int j = 0; j < FN; ++j)
            lh[j] = col0 + (j / 4) * 64 < cols_valid ? hrow + uint32_t(col0 + j * 16 + r16) * 2
                                                        : kOffNone;
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t rowoff = uint32_t(i * 16 + r) * g.Hp * 2;
#pragma unroll
              for (int j = 0; j < FN; ++j)
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16_rne_bits(acc[i][j][r]),
                                                      hrs, lh[j] + rowoff, 0, 0);
            }
        }
        return;
      }
      float* cbase;
      uint32_t ldc;
      if (OP == MOONEP_WGRAD) {
        cbase = (te.wrow < g.E ? g.grad_home + int64_t(te.wrow) * wsz
                               : g.reduce_buf + int64_t(te.wrow - g.E) * wsz) +
                int64_t(m0) * g.Hp + n0;
        ldc = g.Hp;
      } else {
        cbase = g.c + (int64_t(te.rowbase) + m0) * Ndim + n0;
        ldc = Ndim;
      }
      const __amdgpu_buffer_rsrc_t crs = make_rsrc(cbase, clamp_bytes(int64_t(rows_valid) * ldc * 4));
      if constexpr (SWAP) {
        // lane holds row row0 + i*16 + lane%16, columns col0 + j*16 + 4*(lane/16) + (0..3);
        // a 4-column group is all in or all out (the column count is a multiple of 64)
        const uint32_t lrow = uint32_t(row0 + r16) * ldc * 4;
        uint32_t lc[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = col0 + j * 16 + 4 * (lane >> 4);
          lc[j] = col < cols_valid ? lrow + uint32_t(col) * 4 : kOffNone;
        }
        // The += reads run kEpiAhead row blocks ahead of the stores. The compiler keeps
        // buffer loads and stores in program order (it cannot tell that they never
        // overlap), so a read written after the previous block's stores would wait for a
        // whole memory round trip of its own: FM * FN of them in a row per tile.
        constexpr int AHEAD = kEpiAhead < FM ? kEpiAhead : FM;
        floatx4_t old[FM][FN];
        auto read_old = [&](int i) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            old[i][j] = __builtin_bit_cast(
                floatx4_t,
                __builtin_amdgcn_raw_buffer_load_b128(crs, lc[j] + uint32_t(i * 16) * ldc * 4, 0, 0));
        };
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) read_old(i);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i_t, old[i][j] + acc[i][j]),
                                                   crs, lc[j] + uint32_t(i * 16) * ldc * 4, 0, 0);
          if (i + AHEAD < FM) read_old(i + AHEAD);
        }
        return;
      }
      uint32_t lb[FN];
      const uint32_t lane_row = lane_rows * ldc * 4;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = col0 + j * 16 + r16;
        lb[j] = col < cols_valid ? lane_row + uint32_t(col) * 4 : kOffNone;
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t rowoff = uint32_t(i * 16 + r) * ldc * 4;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const uint32_t off = lb[j] + rowoff;
            // through a scalar: a bit cast applied to the vector element itself reads
            // element 0 (clang, gfx950 build)
            const float v = acc[i][j][r];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), crs, off, 0,
                                                  STREAM_OUT ? kStreamStore : 0);
          }
        }
    };
    // WGRAD shifts two 16-row fragments of the tile from each DMA-issuing wavefront to its
    // DMA-free SIMD partner (112 and 144 rows), which otherwise waits at the barrier. A/B
    // at H = 4096, H' = 1408, bit-identical: 2780-2794 -> 2706-2730 us; three fragments
    // gained 0.6% more with twice the register spills. FWD measured 0.9% / 2.4% slower with
    // one / two fragments moved, and DGRAD (all wavefronts issue DMAs) no change with
    // fragments moved either way, so both keep equal halves.
    constexpr int ASYM = WAVES_M == 2 && DW < NW && OP == MOONEP_WGRAD ? 2 : 0;
    // HALFN (calls whose last N-tile is at most half full, such as H' = 1408: 128 of 256
    // columns): on such a tile the wavefronts of the empty half would spend every MFMA on
    // columns that are never stored, and they share SIMDs with each other. Instead the
    // first NW/2 wavefronts (one per SIMD) take the wave tiles of the valid half and the
    // others only keep the ring and the barriers. A separate instance, so that the
    // kernel of every other call keeps its code and registers. A/B, bit-identical: FWD at
    // H = 4096, H' = 1408 -1.6%. Compiled into the shared instance instead it made the
    // FWD at H' = 2048 (no such tiles) 1.5% slower; WGRAD on its own instance was 12%
    // slower (one wavefront per SIMD cannot cover its transposed LDS reads).
    int wm_t = wm, wn_t = wn;
    bool idle = false;
    if constexpr (HALFN && WAVES_N % 2 == 0) {
      if (cols_valid <= BN / 2) {
        idle = wid >= NW / 2;
        wm_t = (wid % (NW / 2)) / (WAVES_N / 2);
        wn_t = wid % (WAVES_N / 2);
      }
    }
    if constexpr (ASYM != 0) {
      if (wm_t == 0) tile(std::integral_constant<int, FM - ASYM>(), 0, wn_t * WN, idle);
      else tile(std::integral_constant<int, FM + ASYM>(), (FM - ASYM) * 16, wn_t * WN, idle);
    } else {
      tile(std::integral_constant<int, FM>(), wm_t * WM, wn_t * WN, idle);
    }
  }
}

// ------------------------------------------------------------------ fp32 kernel
// Compensated dot product (Ogita, Rump and Oishi, "Accurate sum and dot product",
// SIAM J. Sci. Comput. 26(6), 2005, algorithm Dot2): every product is split into its
// rounded value and its exact error by one FMA, every addition into its rounded sum
// and its exact error by Knuth's branch-free two-sum, and the errors are summed on
// the side. The result is as accurate as a dot product evaluated in twice the float32
// precision and then rounded: |err| <= u*|dot| + O(n^2 u^2) * sum|a_i b_i|, with no
// sqrt(n) growth over long reductions. Contraction stays off so that every rounded
// product and sum is the one the error terms describe.
struct Dot2 {
  float p = 0.f, s = 0.f;
  __device__ inline void add(float a, float b) {
#pragma clang fp contract(off)
    const float h = a * b;
    const float r = fmaf(a, b, -h);      // a*b - h exactly
    const float x = p + h;
    const float z = x - p;
    const float q = (p - (x - z)) + (h - z);   // p + h - x exactly
    p = x;
    s = s + (q + r);
  }
  __device__ inline float value() const {
#pragma clang fp contract(off)
    return p + s;
  }
};

// One thread per output element; FWD/DGRAD over tile entries of whole segments.
template <int OP>
__global__ __launch_bounds__(256) void gemm_fp32_kernel(const float* __restrict__ a,
                                                        const float* __restrict__ b, float* c,
                                                        float* grad_home, float* reduce_buf,
                                                        const TileEntry* __restrict__ tiles,
                                                        const int32_t* __restrict__ ntiles, int H,
                                                        int Hp, int E) {
  const int nt = *ntiles;
  const int64_t wsz = int64_t(H) * Hp;
  const int Ndim = OP == MOONEP_DGRAD ? H : Hp;
  const int Kdim = OP == MOONEP_FWD ? H : Hp;
  for (int t = blockIdx.y; t < nt; t += gridDim.y) {
    const TileEntry te = tiles[t];
    if (OP != MOONEP_WGRAD) {
      const int64_t work = int64_t(te.n) * Ndim;
      for (int64_t idx = blockIdx.x * 256 + threadIdx.x; idx < work; idx += int64_t(gridDim.x) * 256) {
        const int m = int(idx / Ndim), n = int(idx % Ndim);
        const float* ar = a + (int64_t(te.rowbase) + m) * Kdim;
        const float* w = b + int64_t(te.wrow) * wsz;
        Dot2 d;
        for (int k = 0; k < Kdim; ++k)
          d.add(ar[k], OP == MOONEP_FWD ? w[int64_t(k) * Hp + n] : w[int64_t(n) * Hp + k]);
        c[(int64_t(te.rowbase) + m) * Ndim + n] = d.value();
      }
    } else {
      float* dst = te.wrow < E ? grad_home + int64_t(te.wrow) * wsz
                               : reduce_buf + int64_t(te.wrow - E) * wsz;
      for (int64_t idx = blockIdx.x * 256 + threadIdx.x; idx < wsz; idx += int64_t(gridDim.x) * 256) {
        const int h = int(idx / Hp), p = int(idx % Hp);
        Dot2 d;
        for (int t2 = 0; t2 < te.n; ++t2)
          d.add(a[(int64_t(te.rowbase) + t2) * H + h], b[(int64_t(te.rowbase) + t2) * Hp + p]);
        dst[idx] += d.value();
      }
    }
  }
}

// fp32 gate/up projection with the SwiGLU fused: one thread per (row, intermediate
// column) forms the gate and the up sums as gemm_fp32_kernel does.
__global__ __launch_bounds__(256) void gemm_fp32_swiglu_kernel(
    const float* __restrict__ a, const float* __restrict__ b, float* __restrict__ act,
    float* __restrict__ h_saved, const TileEntry* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, int H, int Hact) {
  const int nt = *ntiles;
  const int H2 = 2 * Hact;
  const int64_t wsz = int64_t(H) * H2;
  for (int t = blockIdx.y; t < nt; t += gridDim.y) {
    const TileEntry te = tiles[t];
    const int64_t work = int64_t(te.n) * Hact;
    for (int64_t idx = blockIdx.x * 256 + threadIdx.x; idx < work; idx += int64_t(gridDim.x) * 256) {
      const int m = int(idx / Hact), p = int(idx % Hact);
      const int gc = 2 * kSwigluBlock * (p / kSwigluBlock) + p % kSwigluBlock;
      const int64_t row = int64_t(te.rowbase) + m;
      const float* ar = a + row * H;
      const float* w = b + int64_t(te.wrow) * wsz;
      Dot2 dg, du;
      for (int k = 0; k < H; ++k) {
        dg.add(ar[k], w[int64_t(k) * H2 + gc]);
        du.add(ar[k], w[int64_t(k) * H2 + gc + kSwigluBlock]);
      }
      const float sg = dg.value(), su = du.value();
      act[row * Hact + p] = swiglu_f32(sg, su);
      if (h_saved) {
        h_saved[row * H2 + gc] = sg;
        h_saved[row * H2 + gc + kSwigluBlock] = su;
      }
    }
  }
}

// ------------------------------------------------------------------ host
// Compute units of the current device, cached per device. Host threads may call
// concurrently: every store of an entry writes the same value.
static int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// bf16 tile configuration: 256 x 256 output tiles, 8 wavefronts (two per SIMD, so
// one wavefront's waits overlap the other's MFMAs) of 128 x 64, 64-deep k-steps in
// a 2-stage LDS ring (128 KiB), one workgroup per CU. Four wavefronts of 128 x 128
// (a third fewer LDS bytes per flop, and a higher clock) measured 11% slower: with
// one wavefront per SIMD the matrix pipe idles at every wait.
struct TileCfg {
  static constexpr int BM = 256, BN = 256, WAVES_M = 2, WAVES_N = 4, STAGES = 2;
};
// Segment tails of at most kTailRows rows (DGRAD, fused gate/up): 128 x 512 tiles, the same
// 128 x 64 wavefront tile with the 8 wavefronts side by side in N, a 160 KiB
// 2-stage ring (16 KiB + 64 KiB per stage).
// A 256 x 256 tile spends as many MFMAs on a tail of 1..128 rows as on a full one;
// a 128 x 512 tile covers twice the columns for the same MFMAs.
struct TailCfg {
  static constexpr int BM = 128, BN = 512, WAVES_M = 1, WAVES_N = 8, STAGES = 2;
};
constexpr int kTailRows = TailCfg::BM;
// Small calls (FWD and DGRAD with under two rounds of full 256 x 256 tiles over the CUs;
// the fused SwiGLU epilogue needs 64-column wavefront tiles and keeps the large ones):
// most of their operand lines come from HBM, not from another workgroup's L2 fetch, and
// one 64-deep step of lookahead leaves each step waiting for HBM. 256 x 128 tiles (8
// wavefronts of 128 x 32) in a 3-stage ring of 48 KiB steps (144 KiB) keep two steps in
// flight and give the CUs twice as many tiles to balance. Against 128 x 128 tiles in a
// 4-stage ring (three steps of 32 KiB in flight), they read a quarter fewer LDS and DMA
// bytes per flop: 88-91 -> 83-86 us at 32768 slots, H = 1024, H' = 512 (A/B, caches
// flushed; 128 x 256 in 3 stages gave nothing). Every output element gets the same MFMAs
// in the same k order as with the large tiles.
struct SmallCfg {
  static constexpr int BM = 256, BN = 128, WAVES_M = 2, WAVES_N = 4, STAGES = 3;
};

static int64_t full_tiles(const moonep_shape& s, int ncols) {
  return int64_t(s.R) * s.S * s.K / TileCfg::BM * ((ncols + TileCfg::BN - 1) / TileCfg::BN);
}

static bool small_tiles(const moonep_shape& s, int ncols, int cus) {
  return full_tiles(s, ncols) < 2 * int64_t(cus);
}

// Whether segment tails get their own launch (DGRAD and the fused gate/up projection;
// a plain FWD runs them in its 256 x 256 launch). The split halves the MFMAs spent on
// tails, but the tail launch waits for the full-tile launch; a GEMM of under four
// rounds of full tiles is latency-bound, and there the second launch costs more than
// it saves (a layer of 32768 slots, H = 1024, H' = 512: 137 -> 101 us without it).
// Either way every output element gets the same MFMAs in the same k order.
static bool split_tails(const moonep_shape& s, int ncols, int cus) {
  return full_tiles(s, ncols) >= 4 * int64_t(cus);
}

template <int OP, bool SWIGLU, typename C, bool STREAM_OUT = false, bool HALFN = false>
static void launch_cfg(const GemmArgs& g, int cus, hipStream_t strm) {
  gemm_bf16_kernel<OP, C::BM, C::BN, C::WAVES_M, C::WAVES_N, SWIGLU, STREAM_OUT, C::STAGES,
                   HALFN><<<cus, C::WAVES_M * C::WAVES_N * 64, 0, strm>>>(g);
}

// The full-tile list (on the small-tile kernel for a small call), then (FWD and DGRAD,
// when the tails are split off) the tail list on the tail kernel.
// Ops whose 256 x 256 launch takes the HALFN instance when the last N-tile of the call
// is at most half full (plain FWD; WGRAD measured slower with it).
template <int OP, bool SWIGLU>
constexpr bool kHalfnOp = OP == MOONEP_FWD && !SWIGLU;

template <int OP, bool SWIGLU = false, bool STREAM_OUT = false>
static void launch_bf16(GemmArgs g, const TileEntry* tails, const int32_t* ntails,
                        bool tails_apart, bool small, int ncols, int cus, hipStream_t strm) {
  if constexpr (OP != MOONEP_WGRAD && !SWIGLU) {
    if (small) {
      launch_cfg<OP, SWIGLU, SmallCfg, STREAM_OUT>(g, cus, strm);
      return;
    }
  }
  const int last = ncols % TileCfg::BN;   // columns of the call's last N-tile (0: full)
  if (kHalfnOp<OP, SWIGLU> && last > 0 && last <= TileCfg::BN / 2)
    launch_cfg<OP, SWIGLU, TileCfg, STREAM_OUT, kHalfnOp<OP, SWIGLU>>(g, cus, strm);
  else
    launch_cfg<OP, SWIGLU, TileCfg, STREAM_OUT>(g, cus, strm);
  if (OP != MOONEP_WGRAD && tails_apart) {
    g.tiles = tails;
    g.ntiles = ntails;
    if (g.qcnt) g.qcnt += kQueueWords;
    launch_cfg<OP, SWIGLU, TailCfg, STREAM_OUT>(g, cus, strm);
  }
}

}  // namespace moonep

using namespace moonep;

namespace moonep {

// Where one grouped-GEMM call keeps its tile lists and their two counts.
struct GemmLists {
  TileEntry* tiles;
  TileEntry* tails;
  int32_t* ntiles;
  int32_t* ntails;
  int64_t max_tiles, max_tail;
  int32_t* qcnt;   // 2 x kQueueWords tile-queue counters
};

// Argument checks shared by the workspace and the scratch entry points; MOONEP_OK
// with `empty` set when there is nothing to compute.
static int gemm_args(const moonep_shape* shape, int32_t op, const void* a, const void* b,
                     const int32_t* cu_seqlens, float* c, float* grad_home, float* reduce_buf,
                     bool& empty) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (op != MOONEP_FWD && op != MOONEP_DGRAD && op != MOONEP_WGRAD) return MOONEP_EINVAL;
  if (op != MOONEP_FWD && s.mode != MOONEP_TRAIN) return MOONEP_EMODE;
  if (s.H % 64 || s.Hp % 64) return MOONEP_EINVAL;
  if (!aligned16(cu_seqlens)) return MOONEP_EINVAL;
  empty = s.S == 0;
  if (empty) return MOONEP_OK;
  if (!aligned16(a) || !aligned16(b)) return MOONEP_EINVAL;
  if (op == MOONEP_WGRAD) {
    if (!aligned16(grad_home) || (s.B > 0 && !aligned16(reduce_buf))) return MOONEP_EINVAL;
  } else if (!aligned16(c)) {
    return MOONEP_EINVAL;
  }
  return MOONEP_OK;
}

// The tile-list kernel, then the GEMM kernel(s) of `op`, all on `strm`.
static int gemm_launch(const moonep_shape& s, int32_t op, const void* a, const void* b,
                       const int32_t* cu_seqlens, float* c, float* grad_home, float* reduce_buf,
                       const GemmLists& w, hipStream_t strm) {
  const bool bf16 = s.dtype == MOONEP_BF16;
  const bool mtiled = bf16 && op != MOONEP_WGRAD;
  const int cus = device_cus();
  if (cus <= 0) return MOONEP_EHIP;
  const int ncols = op == MOONEP_DGRAD ? s.H : s.Hp;
  const bool small = mtiled && small_tiles(s, ncols, cus);
  // a forward on 256 x 256 tiles of at most 8 N-tiles: the kernel's per-XCD tile queues
  const bool queued_fwd = bf16 && op == MOONEP_FWD && !small && cus % 8 == 0 &&
                          (ncols + TileCfg::BN - 1) / TileCfg::BN <= 8;
  const bool tails_apart = op == MOONEP_DGRAD && mtiled && split_tails(s, ncols, cus);
  gemm_tiles_kernel<<<1, 1024, 0, strm>>>(cu_seqlens, s.R, s.E, s.B, s.S * s.K,
                                          mtiled ? (small ? SmallCfg::BM : TileCfg::BM) : 0,
                                          tails_apart ? kTailRows : 0,
                                          bf16 && op == MOONEP_WGRAD, w.tiles, w.ntiles,
                                          int(w.max_tiles), w.tails, w.ntails, int(w.max_tail),
                                          w.qcnt, queued_fwd ? kTailGroup : 0);
  if (launch_status()) return MOONEP_EHIP;

  if (bf16) {
    GemmArgs g{static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), c, grad_home,
               reduce_buf, w.tiles, w.ntiles, s.H, s.Hp, s.E, nullptr, nullptr, w.qcnt};
    if (op == MOONEP_FWD)
      launch_bf16<MOONEP_FWD>(g, w.tails, w.ntails, tails_apart, small, ncols, cus, strm);
    else if (op == MOONEP_DGRAD && s.Hp <= kStreamOutMaxK)
      launch_bf16<MOONEP_DGRAD, false, true>(g, w.tails, w.ntails, tails_apart, small, ncols,
                                             cus, strm);
    else if (op == MOONEP_DGRAD)
      launch_bf16<MOONEP_DGRAD>(g, w.tails, w.ntails, tails_apart, small, ncols, cus, strm);
    else launch_bf16<MOONEP_WGRAD>(g, w.tails, w.ntails, false, false, ncols, cus, strm);
  } else {
    const dim3 grid(64, 256);
    const float* af = static_cast<const float*>(a);
    const float* bfp = static_cast<const float*>(b);
    if (op == MOONEP_FWD)
      gemm_fp32_kernel<MOONEP_FWD><<<grid, 256, 0, strm>>>(af, bfp, c, grad_home, reduce_buf, w.tiles, w.ntiles, s.H, s.Hp, s.E);
    else if (op == MOONEP_DGRAD)
      gemm_fp32_kernel<MOONEP_DGRAD><<<grid, 256, 0, strm>>>(af, bfp, c, grad_home, reduce_buf, w.tiles, w.ntiles, s.H, s.Hp, s.E);
    else
      gemm_fp32_kernel<MOONEP_WGRAD><<<grid, 256, 0, strm>>>(af, bfp, c, grad_home, reduce_buf, w.tiles, w.ntiles, s.H, s.Hp, s.E);
  }
  return launch_status();
}

static GemmLists ws_lists(void* ws, const WsLayout& w) {
  return GemmLists{ws_ptr<TileEntry>(ws, w.tiles), ws_ptr<TileEntry>(ws, w.tiles_tail),
                   ws_ptr<int32_t>(ws, w.flags) + kFlagTileCount,
                   ws_ptr<int32_t>(ws, w.flags) + kFlagTileCountTail, w.max_tiles, w.max_tail,
                   ws_ptr<int32_t>(ws, w.flags) + kFlagQueue};
}

// ------------------------------------------------------------------ no-alloc scratch
// Tile lists of moonep_grouped_gemm_noalloc live in this file-scope device array, one
// copy per device, held until the process ends. Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): its device
// address is resolved once per device with hipGetSymbolAddress and used from then on.
static __device__ __align__(256) char scratch[MOONEP_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device (nullptr on failure), resolved on
// the first call with that device current and cached per device. Concurrent first
// calls resolve the same address.
static char* scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static std::atomic<char*> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  char* p = cache[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  cache[dev].store(static_cast<char*>(q), std::memory_order_release);
  return static_cast<char*>(q);
}

// Scratch layout of one call: the two list counts (words 0 and 1) and the tile-queue
// counters (words kFlagQueue ..), then the two lists, each 256-byte aligned, sized as the
// workspace sizes them.
struct ScratchLayout {
  size_t tiles, tails, total;
};
static ScratchLayout scratch_layout(const WsLayout& w) {
  ScratchLayout l{};
  l.tiles = 256;
  l.tails = align256(l.tiles + size_t(w.max_tiles) * sizeof(TileEntry));
  l.total = align256(l.tails + size_t(w.max_tail) * sizeof(TileEntry));
  return l;
}

}  // namespace moonep

extern "C" int moonep_grouped_gemm(const moonep_shape* shape, int32_t op, const void* a,
                                   const void* b, const int32_t* cu_seqlens, float* c,
                                   float* grad_home, float* reduce_buf, void* ws, size_t ws_bytes,
                                   void* stream) {
  bool empty = false;
  int st = gemm_args(shape, op, a, b, cu_seqlens, c, grad_home, reduce_buf, empty);
  if (st) return st;
  if (!aligned16(ws)) return MOONEP_EINVAL;
  const WsLayout w = ws_layout(*shape);
  if (ws_bytes < w.total) return MOONEP_EWORKSPACE;
  if (empty) return MOONEP_OK;
  return gemm_launch(*shape, op, a, b, cu_seqlens, c, grad_home, reduce_buf, ws_lists(ws, w),
                     as_stream(stream));
}

extern "C" int moonep_grouped_gemm_noalloc(const moonep_shape* shape, int32_t op, const void* a,
                                           const void* b, const int32_t* cu_seqlens, float* c,
                                           float* grad_home, float* reduce_buf, void* stream) {
  bool empty = false;
  int st = gemm_args(shape, op, a, b, cu_seqlens, c, grad_home, reduce_buf, empty);
  if (st) return st;
  const WsLayout w = ws_layout(*shape);
  const ScratchLayout l = scratch_layout(w);
  if (l.total > MOONEP_NOALLOC_SCRATCH_BYTES) return MOONEP_ELIMIT;
  if (empty) return MOONEP_OK;
  char* base = scratch_ptr();
  if (!base) return MOONEP_EHIP;
  const GemmLists lists{reinterpret_cast<TileEntry*>(base + l.tiles),
                        reinterpret_cast<TileEntry*>(base + l.tails),
                        reinterpret_cast<int32_t*>(base), reinterpret_cast<int32_t*>(base) + 1,
                        w.max_tiles, w.max_tail, reinterpret_cast<int32_t*>(base) + kFlagQueue};
  return gemm_launch(*shape, op, a, b, cu_seqlens, c, grad_home, reduce_buf, lists,
                     as_stream(stream));
}

extern "C" int moonep_grouped_gemm_swiglu(const moonep_shape* shape, const void* xp,
                                          const void* w1_all, const int32_t* cu_seqlens, void* act,
                                          void* h_saved, void* ws, size_t ws_bytes, void* stream) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (s.H % 64 || s.Hp % kSwigluBlock) return MOONEP_EINVAL;
  if (!aligned16(cu_seqlens) || !aligned16(ws)) return MOONEP_EINVAL;
  const WsLayout w = ws_layout(s);
  if (ws_bytes < w.total) return MOONEP_EWORKSPACE;
  if (s.S == 0) return MOONEP_OK;
  if (!aligned16(xp) || !aligned16(w1_all) || !aligned16(act)) return MOONEP_EINVAL;
  if (h_saved && !aligned16(h_saved)) return MOONEP_EINVAL;
  hipStream_t strm = as_stream(stream);
  TileEntry* tiles = ws_ptr<TileEntry>(ws, w.tiles);
  TileEntry* tails = ws_ptr<TileEntry>(ws, w.tiles_tail);
  int32_t* ntiles = ws_ptr<int32_t>(ws, w.flags) + kFlagTileCount;
  int32_t* ntails = ws_ptr<int32_t>(ws, w.flags) + kFlagTileCountTail;
  int32_t* qcnt = ws_ptr<int32_t>(ws, w.flags) + kFlagQueue;
  const bool bf16 = s.dtype == MOONEP_BF16;
  const int cus = device_cus();
  if (cus <= 0) return MOONEP_EHIP;
  const bool tails_apart = bf16 && split_tails(s, 2 * s.Hp, cus);
  gemm_tiles_kernel<<<1, 1024, 0, strm>>>(cu_seqlens, s.R, s.E, s.B, s.S * s.K,
                                          bf16 ? TileCfg::BM : 0, tails_apart ? kTailRows : 0,
                                          false, tiles, ntiles, int(w.max_tiles), tails, ntails,
                                          int(w.max_tail), qcnt, 0);
  if (launch_status()) return MOONEP_EHIP;
  if (bf16) {
    GemmArgs g{static_cast<const uint16_t*>(xp), static_cast<const uint16_t*>(w1_all), nullptr,
               nullptr, nullptr, tiles, ntiles, s.H, 2 * s.Hp, s.E,
               static_cast<uint16_t*>(act), static_cast<uint16_t*>(h_saved), qcnt};
    launch_bf16<MOONEP_FWD, true>(g, tails, ntails, tails_apart, false, 2 * s.Hp, cus, strm);
  } else {
    gemm_fp32_swiglu_kernel<<<dim3(64, 256), 256, 0, strm>>>(
        static_cast<const float*>(xp), static_cast<const float*>(w1_all),
        static_cast<float*>(act), static_cast<float*>(h_saved), tiles, ntiles, s.H, s.Hp);
  }
  return launch_status();
}
