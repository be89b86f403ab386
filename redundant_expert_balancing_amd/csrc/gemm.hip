// Grouped GEMM over the [E+B, H, H'] expert view on gfx950.
//
// Experts are addressed purely by row index and the active rows come only from
// cu_seqlens, which never leaves the device [ai-maestro.online "Moonshot AI
// open-sources MoonEP", section "The memory contract"]. Two launches per call:
//
//   tiles   one workgroup turns cu_seqlens [R, E+B+1] into a compact list of
//           work entries (segment start row, weight row, M offset, length).
//   gemm    a persistent kernel walks entry x N-tile (x M-tile for WGRAD) in an
//           order that keeps the workgroups of one XCD on neighbouring tiles.
//
// bf16 path: v_mfma_f32_32x32x16_bf16, float32 accumulation, operand tiles
// staged through LDS k-contiguous ([rows][BK + 8], the pad keeps 16-byte
// fragment reads conflict-free). Operands stored with k contiguous are copied
// as 16-byte vectors; operands stored with M or N contiguous (the weight in
// FWD, both operands in WGRAD) are loaded as 16-byte vectors and transposed in
// registers before the LDS store. Two LDS stages, one barrier per k-step.
// fp32 path: a plain FMA kernel per output element (tiny layers only).
#include <type_traits>

#include "common.h"

namespace moonep {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;

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

__global__ __launch_bounds__(1024) void gemm_tiles_kernel(const int32_t* __restrict__ cu, int R,
                                                          int E, int B, int SK, int bm,
                                                          TileEntry* __restrict__ tiles,
                                                          int32_t* __restrict__ ntiles,
                                                          int max_tiles) {
  __shared__ int swave[17];
  const int EB = E + B, total = R * EB;
  const int per = (total + 1023) / 1024;
  const int i0 = threadIdx.x * per, i1 = min(total, i0 + per);
  int cnt = 0;
  for (int idx = i0; idx < i1; ++idx) {
    const int q = idx / EB, i = idx % EB;
    const int n = cu[q * (EB + 1) + i + 1] - cu[q * (EB + 1) + i];
    if (n > 0) cnt += bm > 0 ? (n + bm - 1) / bm : 1;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_scan_incl(cnt);
  if (lane == 63) swave[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int x = lane < 16 ? swave[lane] : 0;
    const int xi = wave_scan_incl(x);
    if (lane < 16) swave[lane] = xi - x;
    if (lane == 15) swave[16] = xi;
  }
  __syncthreads();
  int k = swave[w] + incl - cnt;
  for (int idx = i0; idx < i1; ++idx) {
    const int q = idx / EB, i = idx % EB;
    const int c0 = cu[q * (EB + 1) + i];
    const int n = cu[q * (EB + 1) + i + 1] - c0;
    if (n <= 0) continue;
    const int wrow = i < E ? i : E + q * B + (i - E);
    const int step = bm > 0 ? bm : n;
    for (int m0 = 0; m0 < n; m0 += step) {
      if (k < max_tiles) tiles[k] = TileEntry{q * SK + c0, wrow, m0, n};
      ++k;
    }
  }
  if (threadIdx.x == 0) *ntiles = min(swave[16], max_tiles);
}

// ------------------------------------------------------------------ staging
// Operands are read and results written through buffer resources: a 128-bit
// descriptor (base, byte range) in scalar registers plus a 32-bit offset per
// lane. Loads past the range return 0 and stores past it are dropped, which
// zero-fills partial tiles and masks their stores without branches.
typedef int v4i_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcFlags = 0x00020000;   // raw (unswizzled) 32-bit data, gfx9 family
constexpr uint32_t kOffNone = 0x80000000u;  // an offset past every range used here

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcFlags);
}

__device__ inline uint32_t clamp_bytes(int64_t b) {
  return b <= 0 ? 0u : (b >= int64_t(kOffNone) ? kOffNone : uint32_t(b));
}

// k-contiguous operand: ROWS x BK tile; row r at byte offset r*ld*2 of the
// descriptor base; rows past the range read as 0.
template <int ROWS, int BK, int NTHR>
struct StageK {
  static constexpr int VPR = BK / 8;
  static constexpr int PER = ROWS * VPR / NTHR;
  static_assert(ROWS * VPR % NTHR == 0, "tile must split evenly over the threads");
  v4i_t r[PER];
  __device__ inline void load(__amdgpu_buffer_rsrc_t rs, uint32_t ld_bytes) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = threadIdx.x + p * NTHR;
      const int row = v / VPR, kv = v % VPR;
      r[p] = __builtin_amdgcn_raw_buffer_load_b128(rs, row * ld_bytes + kv * 16, 0, 0);
    }
  }
  __device__ inline void store(uint16_t* s) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = threadIdx.x + p * NTHR;
      const int row = v / VPR, kv = v % VPR;
      *reinterpret_cast<v4i_t*>(s + row * (BK + 8) + kv * 8) = r[p];
    }
  }
};

// M/N-contiguous operand: BK x COLS tile, k row i at byte offset i*ld*2, stored to
// LDS transposed as [COLS][BK + 8]. Each thread moves KB k-rows x 8 columns per
// step; consecutive lanes take consecutive k-blocks of one column block, so a
// store instruction covers whole 16-byte chunks of neighbouring LDS rows (no
// bank conflicts) while each k row is still read in whole 128-byte lines.
// Columns at or past cols_valid, and k rows past the range, read as 0.
template <int COLS, int BK, int NTHR>
struct StageMN {
  static constexpr int KB0 = BK * COLS / (8 * NTHR);
  static constexpr int KB = KB0 >= 8 ? 8 : KB0;
  static constexpr int STEPS = BK * COLS / (8 * KB * NTHR);
  static constexpr int KPB = BK / KB;   // k blocks per column block
  static_assert(KB == 2 || KB == 4 || KB == 8, "unsupported transposed staging shape");
  static_assert(STEPS * 8 * KB * NTHR == BK * COLS, "tile must split evenly");
  v4i_t r[STEPS][KB];
  __device__ inline void load(__amdgpu_buffer_rsrc_t rs, uint32_t ld_bytes, int cols_valid) {
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int mb = threadIdx.x + st * NTHR;
      const int kb = mb % KPB, cb = mb / KPB;
      const uint32_t base = cb * 8 < cols_valid ? uint32_t(kb * KB) * ld_bytes + cb * 16 : kOffNone;
#pragma unroll
      for (int i = 0; i < KB; ++i)
        r[st][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + i * ld_bytes, 0, 0);
    }
  }
  __device__ inline void store(uint16_t* s) const {
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int mb = threadIdx.x + st * NTHR;
      const int kb = mb % KPB, cb = mb / KPB;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t o[KB / 2];
#pragma unroll
        for (int j = 0; j < KB / 2; ++j) {
          const uint32_t lo = uint32_t(r[st][2 * j][c >> 1]);
          const uint32_t hi = uint32_t(r[st][2 * j + 1][c >> 1]);
          o[j] = (c & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        uint16_t* dst = s + (cb * 8 + c) * (BK + 8) + kb * KB;
        if constexpr (KB == 2) *reinterpret_cast<uint32_t*>(dst) = o[0];
        else if constexpr (KB == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
        else *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
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
};

template <int OP, int BM, int BN, int BK, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NTHR = WAVES_M * WAVES_N * 64;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int LDK = BK + 8;
  static_assert(FM >= 1 && FN >= 1 && BK % 16 == 0, "tile shape");
  constexpr bool A_MN = OP == MOONEP_WGRAD;  // A stored m-contiguous
  constexpr bool B_MN = OP != MOONEP_DGRAD;  // B stored n-contiguous

  __shared__ __align__(16) uint16_t sA[2][BM * LDK];
  __shared__ __align__(16) uint16_t sB[2][BN * LDK];

  const int Ndim = OP == MOONEP_DGRAD ? g.H : g.Hp;   // columns of C
  const int Kfix = OP == MOONEP_FWD ? g.H : g.Hp;     // FWD/DGRAD reduction length
  const int NT = (Ndim + BN - 1) / BN;
  const int MT = OP == MOONEP_WGRAD ? (g.H + BM - 1) / BM : 1;
  const int64_t total = int64_t(*g.ntiles) * MT * NT;
  const int64_t wsz = int64_t(g.H) * g.Hp;
  const uint32_t lda_b = uint32_t(OP == MOONEP_DGRAD ? g.Hp : g.H) * 2;   // bytes per A row
  const uint32_t ldb_b = uint32_t(g.Hp) * 2;                              // bytes per B row

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int r32 = lane & 31, kh = (lane >> 5) * 8;

  // XCD-aware order: the workgroups of one XCD take a contiguous run of tiles.
  const int G = gridDim.x;
  const int slot = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;

  typename std::conditional<A_MN, StageMN<BM, BK, NTHR>, StageK<BM, BK, NTHR>>::type stA;
  typename std::conditional<B_MN, StageMN<BN, BK, NTHR>, StageK<BN, BK, NTHR>>::type stB;

  for (int64_t tau = slot; tau < total; tau += G) {
    const int64_t ent = tau / (int64_t(MT) * NT);
    const int rem = int(tau % (int64_t(MT) * NT));
    const int mt = rem / NT, nt = rem % NT;
    const TileEntry te = g.tiles[ent];
    const int n0 = nt * BN;
    const int cols_valid = min(BN, Ndim - n0);
    int m0, rows_valid, kdim;
    if (OP == MOONEP_WGRAD) {
      m0 = mt * BM;
      rows_valid = min(BM, g.H - m0);
      kdim = te.n;
    } else {
      m0 = te.m0;
      rows_valid = min(BM, te.n - te.m0);
      kdim = Kfix;
    }
    // operand bases at k = 0 of this tile
    const uint16_t* abase;
    const uint16_t* bbase;
    if (OP == MOONEP_FWD) {
      abase = g.a + (int64_t(te.rowbase) + m0) * g.H;
      bbase = g.b + int64_t(te.wrow) * wsz + n0;
    } else if (OP == MOONEP_DGRAD) {
      abase = g.a + (int64_t(te.rowbase) + m0) * g.Hp;
      bbase = g.b + int64_t(te.wrow) * wsz + int64_t(n0) * g.Hp;
    } else {
      abase = g.a + int64_t(te.rowbase) * g.H + m0;
      bbase = g.b + int64_t(te.rowbase) * g.Hp + n0;
    }

    floatx16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int kiters = (kdim + BK - 1) / BK;
    auto load_stage = [&](int kt) {
      const int k0 = kt * BK;
      if constexpr (A_MN) {
        stA.load(make_rsrc(abase + int64_t(k0) * g.H, clamp_bytes(int64_t(kdim - k0) * lda_b)),
                 lda_b, rows_valid);
      } else {
        stA.load(make_rsrc(abase + k0, clamp_bytes(int64_t(rows_valid) * lda_b)), lda_b);
      }
      if constexpr (B_MN) {
        stB.load(make_rsrc(bbase + int64_t(k0) * g.Hp, clamp_bytes(int64_t(kdim - k0) * ldb_b)),
                 ldb_b, cols_valid);
      } else {
        stB.load(make_rsrc(bbase + k0, clamp_bytes(int64_t(cols_valid) * ldb_b)), ldb_b);
      }
    };

    if (kiters > 0) {
      load_stage(0);
      stA.store(sA[0]);
      stB.store(sB[0]);
    }
    __syncthreads();
    for (int kt = 0; kt < kiters; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < kiters) load_stage(kt + 1);
      const uint16_t* pa = sA[cur] + (wm * WM + r32) * LDK + kh;
      const uint16_t* pb = sB[cur] + (wn * WN + r32) * LDK + kh;
      // fragments of the next 16-wide k slice are read while this slice's MFMAs run
      bf16x8_t af[2][FM], bfr[2][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[0][i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * LDK);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[0][j] = *reinterpret_cast<const bf16x8_t*>(pb + j * 32 * LDK);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int c = ks & 1;
        if (ks + 1 < BK / 16) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
            af[c ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * LDK + (ks + 1) * 16);
#pragma unroll
          for (int j = 0; j < FN; ++j)
            bfr[c ^ 1][j] = *reinterpret_cast<const bf16x8_t*>(pb + j * 32 * LDK + (ks + 1) * 16);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[c][i], bfr[c][j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < kiters) {
        stA.store(sA[cur ^ 1]);
        stB.store(sB[cur ^ 1]);
      }
      __syncthreads();
    }

    // epilogue: lane holds column (lane % 32) and rows 8*(r/4) + 4*(lane/32) + r%4
    // of each 32 x 32 block; rows past rows_valid fall outside the range.
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
    // per-lane byte offset of each column block (columns past cols_valid fall
    // outside the range); the row part of the offset is the same for every lane
    uint32_t lb[FN];
    const uint32_t lane_row = uint32_t(wm * WM + (lane >> 5) * 4) * ldc * 4;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = wn * WN + j * 32 + r32;
      lb[j] = col < cols_valid ? lane_row + uint32_t(col) * 4 : kOffNone;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t rowoff = uint32_t(i * 32 + (r >> 2) * 8 + (r & 3)) * ldc * 4;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint32_t off = lb[j] + rowoff;
          float v = acc[i][j][r];
          if (OP == MOONEP_WGRAD)
            v += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(crs, off, 0, 0));
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), crs, off, 0, 0);
        }
      }
  }
}

// ------------------------------------------------------------------ fp32 kernel
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
        float s = 0.f;
        for (int k = 0; k < Kdim; ++k)
          s = fmaf(ar[k], OP == MOONEP_FWD ? w[int64_t(k) * Hp + n] : w[int64_t(n) * Hp + k], s);
        c[(int64_t(te.rowbase) + m) * Ndim + n] = s;
      }
    } else {
      float* dst = te.wrow < E ? grad_home + int64_t(te.wrow) * wsz
                               : reduce_buf + int64_t(te.wrow - E) * wsz;
      for (int64_t idx = blockIdx.x * 256 + threadIdx.x; idx < wsz; idx += int64_t(gridDim.x) * 256) {
        const int h = int(idx / Hp), p = int(idx % Hp);
        float s = 0.f;
        for (int t2 = 0; t2 < te.n; ++t2)
          s = fmaf(a[(int64_t(te.rowbase) + t2) * H + h], b[(int64_t(te.rowbase) + t2) * Hp + p], s);
        dst[idx] += s;
      }
    }
  }
}

// ------------------------------------------------------------------ host
static int device_cus() {
  static int cached_dev = -1, cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev != cached_dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached_dev = dev;
    cached = n;
  }
  return cached;
}

// bf16 tile configuration: 256 x 256 output tile, 4 wavefronts of 128 x 128,
// k-steps of 64, two LDS stages (147 KB), one workgroup per CU.
template <int OP>
struct TileCfg {
  static constexpr int BM = 256, BN = 256, BK = 64, WAVES_M = 2, WAVES_N = 2;
};
constexpr int kBlocksPerCU = 1;

template <int OP>
static void launch_bf16(const GemmArgs& g, int grid, hipStream_t strm) {
  using C = TileCfg<OP>;
  gemm_bf16_kernel<OP, C::BM, C::BN, C::BK, C::WAVES_M, C::WAVES_N>
      <<<grid, C::WAVES_M * C::WAVES_N * 64, 0, strm>>>(g);
}

}  // namespace moonep

using namespace moonep;

extern "C" int moonep_grouped_gemm(const moonep_shape* shape, int32_t op, const void* a,
                                   const void* b, const int32_t* cu_seqlens, float* c,
                                   float* grad_home, float* reduce_buf, void* ws, size_t ws_bytes,
                                   void* stream) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (op != MOONEP_FWD && op != MOONEP_DGRAD && op != MOONEP_WGRAD) return MOONEP_EINVAL;
  if (op != MOONEP_FWD && s.mode != MOONEP_TRAIN) return MOONEP_EMODE;
  if (s.H % 64 || s.Hp % 64) return MOONEP_EINVAL;
  if (!aligned16(cu_seqlens) || !aligned16(ws)) return MOONEP_EINVAL;
  const WsLayout w = ws_layout(s);
  if (ws_bytes < w.total) return MOONEP_EWORKSPACE;
  if (s.S == 0) return MOONEP_OK;
  if (!aligned16(a) || !aligned16(b)) return MOONEP_EINVAL;
  if (op == MOONEP_WGRAD) {
    if (!aligned16(grad_home) || (s.B > 0 && !aligned16(reduce_buf))) return MOONEP_EINVAL;
  } else if (!aligned16(c)) {
    return MOONEP_EINVAL;
  }
  hipStream_t strm = as_stream(stream);
  TileEntry* tiles = ws_ptr<TileEntry>(ws, w.tiles);
  int32_t* ntiles = ws_ptr<int32_t>(ws, w.flags) + kFlagTileCount;
  const bool bf16 = s.dtype == MOONEP_BF16;
  const int bm = (op == MOONEP_WGRAD || !bf16) ? 0 : TileCfg<MOONEP_FWD>::BM;
  gemm_tiles_kernel<<<1, 1024, 0, strm>>>(cu_seqlens, s.R, s.E, s.B, s.S * s.K, bm, tiles, ntiles,
                                          int(w.max_tiles));
  if (launch_status()) return MOONEP_EHIP;

  if (bf16) {
    const int cus = device_cus();
    if (cus <= 0) return MOONEP_EHIP;
    GemmArgs g{static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), c, grad_home,
               reduce_buf, tiles, ntiles, s.H, s.Hp, s.E};
    const int grid = cus * kBlocksPerCU;
    if (op == MOONEP_FWD) launch_bf16<MOONEP_FWD>(g, grid, strm);
    else if (op == MOONEP_DGRAD) launch_bf16<MOONEP_DGRAD>(g, grid, strm);
    else launch_bf16<MOONEP_WGRAD>(g, grid, strm);
  } else {
    const dim3 grid(64, 256);
    const float* af = static_cast<const float*>(a);
    const float* bfp = static_cast<const float*>(b);
    if (op == MOONEP_FWD)
      gemm_fp32_kernel<MOONEP_FWD><<<grid, 256, 0, strm>>>(af, bfp, c, grad_home, reduce_buf, tiles, ntiles, s.H, s.Hp, s.E);
    else if (op == MOONEP_DGRAD)
      gemm_fp32_kernel<MOONEP_DGRAD><<<grid, 256, 0, strm>>>(af, bfp, c, grad_home, reduce_buf, tiles, ntiles, s.H, s.Hp, s.E);
    else
      gemm_fp32_kernel<MOONEP_WGRAD><<<grid, 256, 0, strm>>>(af, bfp, c, grad_home, reduce_buf, tiles, ntiles, s.H, s.Hp, s.E);
  }
  return launch_status();
}
