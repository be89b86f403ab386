// HBM-bound data movement of the balanced MoE layer on gfx950: fused permute
// (dispatch), fused unpermute (combine), prefetch of replica weights and the
// fold of replica gradients (reduce_grad). All moves are 16-byte vectors with
// consecutive lanes on consecutive addresses of a row; per-token slot indices
// and gates are uniform across a workgroup, staged once in LDS.
//
// [ai-maestro.online "Moonshot AI open-sources MoonEP": "The core idea: dynamic
// redundant experts" (zero copy: tokens written straight to their
// expert-grouped positions; replicas prefetched before expert compute, their
// gradients sent home in backward), "The memory contract" (prefetch slots
// filled by prefetch_weight; reduce_grad adds the slots of a rank's experts from
// every rank into its parameter grad and zeroes the consumed slots).]
#include "common.h"

namespace moonep {

constexpr int kMoveThreads = 256;
constexpr int kMaxK = 32;

// Two bf16 values (one 32-bit word) scaled by g in float32, rounded once.
__device__ inline uint32_t scale_bf16x2(uint32_t w, float g) {
  const float lo = __uint_as_float(w << 16) * g;
  const float hi = __uint_as_float(w & 0xFFFF0000u) * g;
  return bf16_rne_bits(lo) | (bf16_rne_bits(hi) << 16);
}

__device__ inline uint4 scale_vec(uint4 v, float g, bool bf16) {
  if (bf16) {
    v.x = scale_bf16x2(v.x, g); v.y = scale_bf16x2(v.y, g);
    v.z = scale_bf16x2(v.z, g); v.w = scale_bf16x2(v.w, g);
  } else {
    v.x = __float_as_uint(__uint_as_float(v.x) * g);
    v.y = __float_as_uint(__uint_as_float(v.y) * g);
    v.z = __float_as_uint(__uint_as_float(v.z) * g);
    v.w = __float_as_uint(__uint_as_float(v.w) * g);
  }
  return v;
}

typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

__device__ inline v4u_t scale_v4u(v4u_t v, float g, bool bf16) {
  uint4 u = make_uint4(v.x, v.y, v.z, v.w);
  u = scale_vec(u, g, bf16);
  return v4u_t{u.x, u.y, u.z, u.w};
}

// One workgroup per token: each thread loads one 16-byte vector of the row, then
// writes it to the K destinations, and moves on to the next 256 vectors. Plain
// stores: non-temporal ones measured 7% slower for this write-heavy scatter; two or
// four vectors per thread in flight measured 1-4% slower.
template <bool GATED, bool BF16>
__global__ __launch_bounds__(kMoveThreads) void dispatch_kernel(
    const v4u_t* __restrict__ src, int nvec, int N, int K, const int32_t* __restrict__ slot_map,
    const float* __restrict__ gates, v4u_t* __restrict__ dst, int64_t ndst) {
  __shared__ int32_t s_slot[kMaxK];
  __shared__ float s_gate[kMaxK];
  for (int g = blockIdx.x; g < N; g += gridDim.x) {
    if (threadIdx.x < K) {
      const int d = slot_map[int64_t(g) * K + threadIdx.x];
      s_slot[threadIdx.x] = (d >= 0 && d < ndst) ? d : -1;
      if (GATED) s_gate[threadIdx.x] = gates[int64_t(g) * K + threadIdx.x];
    }
    __syncthreads();
    const v4u_t* row = src + int64_t(g) * nvec;
    for (int v = threadIdx.x; v < nvec; v += kMoveThreads) {
      const v4u_t val = row[v];
      for (int k = 0; k < K; ++k) {
        const int d = s_slot[k];
        if (d < 0) continue;
        dst[int64_t(d) * nvec + v] = GATED ? scale_v4u(val, s_gate[k], BF16) : val;
      }
    }
    __syncthreads();
  }
}

// One workgroup per token: y[g] = sum over k ascending of w_k * src[slot(g,k)].
// Each thread issues all K x VPT loads before the multiply-adds; the expert
// outputs are read exactly once, so the loads are non-temporal.
template <bool GATED, int KC, int VPT>  // KC > 0: K known at compile time
__global__ __launch_bounds__(kMoveThreads) void combine_kernel(
    const v4f_t* __restrict__ src, int nvec, int N, int Kr, const int32_t* __restrict__ slot_map,
    const float* __restrict__ gates, v4f_t* __restrict__ dst, int64_t nsrc) {
  __shared__ int32_t s_slot[kMaxK];
  __shared__ float s_gate[kMaxK];
  const int K = KC > 0 ? KC : Kr;
  for (int g = blockIdx.x; g < N; g += gridDim.x) {
    if (threadIdx.x < K) {
      const int d = slot_map[int64_t(g) * K + threadIdx.x];
      s_slot[threadIdx.x] = (d >= 0 && d < nsrc) ? d : -1;
      s_gate[threadIdx.x] = GATED ? gates[int64_t(g) * K + threadIdx.x] : 1.0f;
    }
    __syncthreads();
    for (int v0 = 0; v0 < nvec; v0 += VPT * kMoveThreads) {
      v4f_t acc[VPT];
#pragma unroll
      for (int i = 0; i < VPT; ++i) acc[i] = v4f_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (KC > 0) {
        v4f_t x[KC][VPT];
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          const int d = s_slot[k];
#pragma unroll
          for (int i = 0; i < VPT; ++i) {
            const int v = v0 + i * kMoveThreads + threadIdx.x;
            x[k][i] = (d >= 0 && v < nvec) ? __builtin_nontemporal_load(src + int64_t(d) * nvec + v)
                                           : v4f_t{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          const float w = s_gate[k];
#pragma unroll
          for (int i = 0; i < VPT; ++i) {
            acc[i].x = fmaf(w, x[k][i].x, acc[i].x); acc[i].y = fmaf(w, x[k][i].y, acc[i].y);
            acc[i].z = fmaf(w, x[k][i].z, acc[i].z); acc[i].w = fmaf(w, x[k][i].w, acc[i].w);
          }
        }
      } else {
        for (int k = 0; k < K; ++k) {
          const int d = s_slot[k];
          if (d < 0) continue;
          const float w = s_gate[k];
#pragma unroll
          for (int i = 0; i < VPT; ++i) {
            const int v = v0 + i * kMoveThreads + threadIdx.x;
            if (v < nvec) {
              const v4f_t y = __builtin_nontemporal_load(src + int64_t(d) * nvec + v);
              acc[i].x = fmaf(w, y.x, acc[i].x); acc[i].y = fmaf(w, y.y, acc[i].y);
              acc[i].z = fmaf(w, y.z, acc[i].z); acc[i].w = fmaf(w, y.w, acc[i].w);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int v = v0 + i * kMoveThreads + threadIdx.x;
        if (v < nvec) dst[int64_t(g) * nvec + v] = acc[i];
      }
    }
    __syncthreads();
  }
}

// Copy home rows into used prefetch slots; every workgroup takes a stripe of
// every used slot, so the launch never depends on how many slots are used.
__global__ __launch_bounds__(kMoveThreads) void prefetch_kernel(const int32_t* __restrict__ replica,
                                                                int RB, int E,
                                                                uint4* __restrict__ w_all,
                                                                int64_t vpe) {
  const int64_t stride = int64_t(gridDim.x) * kMoveThreads;
  const int64_t i0 = int64_t(blockIdx.x) * kMoveThreads + threadIdx.x;
  for (int s = 0; s < RB; ++s) {
    const int e = replica[s];
    if (e < 0 || e >= E) continue;
    const uint4* from = w_all + int64_t(e) * vpe;
    uint4* to = w_all + (int64_t(E) + s) * vpe;
    for (int64_t i = i0; i < vpe; i += stride) to[i] = from[i];
  }
}

// grad_home[e] += sum of the slots holding e, in slot order (q asc, j asc);
// the slots are zeroed. LDS holds the slot list, each slot's next slot of the
// same expert, and the first slot of every replicated expert.
__global__ __launch_bounds__(kMoveThreads) void reduce_grad_kernel(
    const int32_t* __restrict__ replica, int RB, int E, float4* __restrict__ reduce_buf,
    float4* __restrict__ grad_home, int64_t vpe) {
  extern __shared__ int32_t lds[];
  int32_t* rep = lds;
  int32_t* nxt = lds + RB;
  int32_t* firsts = lds + 2 * RB;
  __shared__ int nfirst;
  if (threadIdx.x == 0) nfirst = 0;
  for (int s = threadIdx.x; s < RB; s += kMoveThreads) {
    const int e = replica[s];
    rep[s] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
  for (int s = threadIdx.x; s < RB; s += kMoveThreads) {
    const int e = rep[s];
    int n = -1;
    bool first = e >= 0;
    if (e >= 0) {
      for (int s2 = s + 1; s2 < RB; ++s2)
        if (rep[s2] == e) { n = s2; break; }
      for (int s2 = 0; s2 < s && first; ++s2)
        if (rep[s2] == e) first = false;
    }
    nxt[s] = n;
    if (first) firsts[atomicAdd(&nfirst, 1)] = s;
  }
  __syncthreads();
  const int nf = nfirst;
  const int64_t stride = int64_t(gridDim.x) * kMoveThreads;
  const int64_t i0 = int64_t(blockIdx.x) * kMoveThreads + threadIdx.x;
  for (int f = 0; f < nf; ++f) {
    const int s0 = firsts[f];
    const int e = rep[s0];
    float4* gh = grad_home + int64_t(e) * vpe;
    for (int64_t i = i0; i < vpe; i += stride) {
      float4 acc = gh[i];
      for (int s = s0; s >= 0; s = nxt[s]) {
        float4* rb = reduce_buf + int64_t(s) * vpe + i;
        const float4 v = *rb;
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        *rb = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      gh[i] = acc;
    }
  }
}

inline int grid_for(int64_t work, int cap) {
  return int(work < cap ? (work > 0 ? work : 1) : cap);
}

}  // namespace moonep

using namespace moonep;

extern "C" int moonep_dispatch(const moonep_shape* shape, int32_t width, const void* src,
                               const int32_t* slot_map, const float* gates, void* dst,
                               void* stream) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  const int eb = elem_bytes(s);
  if (width != s.H && width != s.Hp) return MOONEP_EINVAL;
  const int N = s.R * s.S;
  if (N == 0) return MOONEP_OK;
  if (!aligned16(src) || !aligned16(slot_map) || !aligned16(dst)) return MOONEP_EINVAL;
  if (gates && !aligned16(gates)) return MOONEP_EINVAL;
  const int nvec = width * eb / 16;
  const int64_t ndst = int64_t(N) * s.K;
  const int grid = grid_for(N, 1 << 20);
  hipStream_t strm = as_stream(stream);
  const v4u_t* sv = static_cast<const v4u_t*>(src);
  v4u_t* dv = static_cast<v4u_t*>(dst);
#define MOONEP_DISPATCH(G, B) \
  dispatch_kernel<G, B><<<grid, kMoveThreads, 0, strm>>>(sv, nvec, N, s.K, slot_map, gates, dv, ndst)
  if (!gates) MOONEP_DISPATCH(false, true);
  else if (s.dtype == MOONEP_BF16) MOONEP_DISPATCH(true, true);
  else MOONEP_DISPATCH(true, false);
#undef MOONEP_DISPATCH
  return launch_status();
}

template <bool GATED, int VPT>
static void launch_combine(int grid, hipStream_t strm, const v4f_t* src, int nvec, int N, int K,
                           const int32_t* slot_map, const float* gates, v4f_t* dst,
                           int64_t nsrc) {
#define MOONEP_COMBINE(KC) \
  combine_kernel<GATED, KC, VPT><<<grid, kMoveThreads, 0, strm>>>(src, nvec, N, K, slot_map, gates, dst, nsrc)
  switch (K) {
    case 1: MOONEP_COMBINE(1); break;
    case 2: MOONEP_COMBINE(2); break;
    case 4: MOONEP_COMBINE(4); break;
    case 6: MOONEP_COMBINE(6); break;
    case 8: MOONEP_COMBINE(8); break;
    default: MOONEP_COMBINE(0); break;
  }
#undef MOONEP_COMBINE
}

extern "C" int moonep_combine(const moonep_shape* shape, int32_t width, const float* src,
                              const int32_t* slot_map, const float* gates, float* dst,
                              void* stream) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (width != s.H && width != s.Hp) return MOONEP_EINVAL;
  if (width % 4) return MOONEP_EINVAL;
  const int N = s.R * s.S;
  if (N == 0) return MOONEP_OK;
  if (!aligned16(src) || !aligned16(slot_map) || !aligned16(dst)) return MOONEP_EINVAL;
  if (gates && !aligned16(gates)) return MOONEP_EINVAL;
  const int nvec = width / 4;
  const int grid = grid_for(N, 1 << 20);
  hipStream_t strm = as_stream(stream);
  const v4f_t* sv = reinterpret_cast<const v4f_t*>(src);
  v4f_t* dv = reinterpret_cast<v4f_t*>(dst);
  const int64_t nsrc = int64_t(N) * s.K;
  const bool two = nvec > kMoveThreads;   // two vectors per thread for long rows
  if (gates) {
    if (two) launch_combine<true, 2>(grid, strm, sv, nvec, N, s.K, slot_map, gates, dv, nsrc);
    else launch_combine<true, 1>(grid, strm, sv, nvec, N, s.K, slot_map, gates, dv, nsrc);
  } else {
    if (two) launch_combine<false, 2>(grid, strm, sv, nvec, N, s.K, slot_map, nullptr, dv, nsrc);
    else launch_combine<false, 1>(grid, strm, sv, nvec, N, s.K, slot_map, nullptr, dv, nsrc);
  }
  return launch_status();
}

extern "C" int moonep_prefetch_weight(const moonep_shape* shape, const int32_t* replica_expert,
                                      void* w_all, void* stream) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (s.B == 0) return MOONEP_OK;
  if (!aligned16(replica_expert) || !aligned16(w_all)) return MOONEP_EINVAL;
  const int64_t vpe = int64_t(s.H) * s.Hp * elem_bytes(s) / 16;
  const int grid = grid_for((vpe + kMoveThreads - 1) / kMoveThreads, 2048);
  prefetch_kernel<<<grid, kMoveThreads, 0, as_stream(stream)>>>(
      replica_expert, s.R * s.B, s.E, static_cast<uint4*>(w_all), vpe);
  return launch_status();
}

extern "C" int moonep_reduce_grad(const moonep_shape* shape, const int32_t* replica_expert,
                                  float* reduce_buf, float* grad_home, void* stream) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (s.mode != MOONEP_TRAIN) return MOONEP_EMODE;
  if (s.B == 0) return MOONEP_OK;
  if (!aligned16(replica_expert) || !aligned16(reduce_buf) || !aligned16(grad_home))
    return MOONEP_EINVAL;
  const int RB = s.R * s.B;
  const int64_t vpe = int64_t(s.H) * s.Hp / 4;
  const int grid = grid_for((vpe + kMoveThreads - 1) / kMoveThreads, 2048);
  reduce_grad_kernel<<<grid, kMoveThreads, size_t(3) * RB * 4, as_stream(stream)>>>(
      replica_expert, RB, s.E, reinterpret_cast<float4*>(reduce_buf),
      reinterpret_cast<float4*>(grad_home), vpe);
  return launch_status();
}
