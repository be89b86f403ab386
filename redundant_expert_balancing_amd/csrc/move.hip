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

__device__ inline uint32_t bf16_rne_bits(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);  // round to nearest, ties to even
  return b >> 16;
}

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

// One workgroup per token: read the row once, write it to its K destinations.
template <bool GATED, bool BF16>
__global__ __launch_bounds__(kMoveThreads) void dispatch_kernel(
    const uint4* __restrict__ src, int nvec, int N, int K, const int32_t* __restrict__ slot_map,
    const float* __restrict__ gates, uint4* __restrict__ dst, int64_t ndst) {
  __shared__ int32_t s_slot[kMaxK];
  __shared__ float s_gate[kMaxK];
  for (int g = blockIdx.x; g < N; g += gridDim.x) {
    if (threadIdx.x < K) {
      s_slot[threadIdx.x] = slot_map[int64_t(g) * K + threadIdx.x];
      if (GATED) s_gate[threadIdx.x] = gates[int64_t(g) * K + threadIdx.x];
    }
    __syncthreads();
    const uint4* row = src + int64_t(g) * nvec;
    for (int v = threadIdx.x; v < nvec; v += kMoveThreads) {
      const uint4 val = row[v];
      for (int k = 0; k < K; ++k) {
        const int d = s_slot[k];
        if (d < 0 || d >= ndst) continue;
        dst[int64_t(d) * nvec + v] = GATED ? scale_vec(val, s_gate[k], BF16) : val;
      }
    }
    __syncthreads();
  }
}

// One workgroup per token: y[g] = sum over k ascending of w_k * src[slot(g,k)].
template <bool GATED, int KC>  // KC > 0: K known at compile time
__global__ __launch_bounds__(kMoveThreads) void combine_kernel(
    const float4* __restrict__ src, int nvec, int N, int Kr, const int32_t* __restrict__ slot_map,
    const float* __restrict__ gates, float4* __restrict__ dst, int64_t nsrc) {
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
    for (int v = threadIdx.x; v < nvec; v += kMoveThreads) {
      float4 x[KC > 0 ? KC : 1];
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      if (KC > 0) {
#pragma unroll
        for (int k = 0; k < (KC > 0 ? KC : 1); ++k) {
          const int d = s_slot[k];
          x[k] = d >= 0 ? src[int64_t(d) * nvec + v] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < (KC > 0 ? KC : 1); ++k) {
          const float w = s_gate[k];
          acc.x = fmaf(w, x[k].x, acc.x); acc.y = fmaf(w, x[k].y, acc.y);
          acc.z = fmaf(w, x[k].z, acc.z); acc.w = fmaf(w, x[k].w, acc.w);
        }
      } else {
        for (int k = 0; k < K; ++k) {
          const int d = s_slot[k];
          if (d < 0) continue;
          const float4 y = src[int64_t(d) * nvec + v];
          const float w = s_gate[k];
          acc.x = fmaf(w, y.x, acc.x); acc.y = fmaf(w, y.y, acc.y);
          acc.z = fmaf(w, y.z, acc.z); acc.w = fmaf(w, y.w, acc.w);
        }
      }
      dst[int64_t(g) * nvec + v] = acc;
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
  const uint4* sv = static_cast<const uint4*>(src);
  uint4* dv = static_cast<uint4*>(dst);
  if (!gates)
    dispatch_kernel<false, true><<<grid, kMoveThreads, 0, strm>>>(sv, nvec, N, s.K, slot_map,
                                                                 nullptr, dv, ndst);
  else if (s.dtype == MOONEP_BF16)
    dispatch_kernel<true, true><<<grid, kMoveThreads, 0, strm>>>(sv, nvec, N, s.K, slot_map,
                                                                gates, dv, ndst);
  else
    dispatch_kernel<true, false><<<grid, kMoveThreads, 0, strm>>>(sv, nvec, N, s.K, slot_map,
                                                                 gates, dv, ndst);
  return launch_status();
}

template <bool GATED>
static void launch_combine(int grid, hipStream_t strm, const float4* src, int nvec, int N, int K,
                           const int32_t* slot_map, const float* gates, float4* dst,
                           int64_t nsrc) {
  switch (K) {
    case 1: combine_kernel<GATED, 1><<<grid, kMoveThreads, 0, strm>>>(src, nvec, N, K, slot_map, gates, dst, nsrc); break;
    case 2: combine_kernel<GATED, 2><<<grid, kMoveThreads, 0, strm>>>(src, nvec, N, K, slot_map, gates, dst, nsrc); break;
    case 4: combine_kernel<GATED, 4><<<grid, kMoveThreads, 0, strm>>>(src, nvec, N, K, slot_map, gates, dst, nsrc); break;
    case 6: combine_kernel<GATED, 6><<<grid, kMoveThreads, 0, strm>>>(src, nvec, N, K, slot_map, gates, dst, nsrc); break;
    case 8: combine_kernel<GATED, 8><<<grid, kMoveThreads, 0, strm>>>(src, nvec, N, K, slot_map, gates, dst, nsrc); break;
    default: combine_kernel<GATED, 0><<<grid, kMoveThreads, 0, strm>>>(src, nvec, N, K, slot_map, gates, dst, nsrc); break;
  }
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
  const float4* sv = reinterpret_cast<const float4*>(src);
  float4* dv = reinterpret_cast<float4*>(dst);
  const int64_t nsrc = int64_t(N) * s.K;
  if (gates)
    launch_combine<true>(grid, strm, sv, nvec, N, s.K, slot_map, gates, dv, nsrc);
  else
    launch_combine<false>(grid, strm, sv, nvec, N, s.K, slot_map, nullptr, dv, nsrc);
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
