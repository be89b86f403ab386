// SwiGLU between the two projections of the expert FFN on gfx950, forward and
// backward, as standalone HBM-bound passes over the slot buffer. (The forward
// also runs fused into the gate/up grouped GEMM's epilogue, gemm.hip, through
// the same swiglu_f32.)
//
// The pages give the per-projection weight contract and the intermediate size
// H' of the expert FFN, not its activation [ai-maestro.online "Moonshot AI
// open-sources MoonEP", section "The memory contract"]; the gated SiLU form is
// this library's reading. Gate and up columns are interleaved in 32-column
// blocks, so 4 consecutive intermediate columns are 4 consecutive gate columns
// and, 32 further, 4 consecutive up columns: one 16-byte float32 vector each.
#include "common.h"

namespace moonep {

constexpr int kFfnThreads = 256;
typedef float v4f_t __attribute__((ext_vector_type(4)));

// element offset, within a [.., 2H'] row, of the gate of intermediate column p
__device__ inline int gate_col(int p) {
  return 2 * kSwigluBlock * (p / kSwigluBlock) + p % kSwigluBlock;
}

template <bool BF16>
__device__ inline v4f_t load4(const void* base, int64_t idx) {
  if (BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return v4f_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
  }
  return *reinterpret_cast<const v4f_t*>(static_cast<const float*>(base) + idx);
}

template <bool BF16>
__device__ inline void store4(void* base, int64_t idx, v4f_t v) {
  if (BF16) {
    uint2 w;
    w.x = bf16_rne_bits(v.x) | (bf16_rne_bits(v.y) << 16);
    w.y = bf16_rne_bits(v.z) | (bf16_rne_bits(v.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = w;
  } else {
    *reinterpret_cast<v4f_t*>(static_cast<float*>(base) + idx) = v;
  }
}

// One thread per 4 intermediate columns of one row: act = swiglu(gate, up),
// optionally h rounded to dtype for the backward pass.
template <bool BF16, bool SAVE>
__global__ __launch_bounds__(kFfnThreads) void swiglu_kernel(const float* __restrict__ h,
                                                             int64_t rows, int Hp,
                                                             void* __restrict__ act,
                                                             void* __restrict__ h_saved) {
  const int q4 = Hp / 4;
  const int64_t total = rows * q4;
  for (int64_t i = blockIdx.x * int64_t(kFfnThreads) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * kFfnThreads) {
    const int64_t r = i / q4;
    const int p = int(i - r * q4) * 4;
    const int64_t gc = r * 2 * Hp + gate_col(p);
    const v4f_t g = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(h + gc));
    const v4f_t u = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(h + gc + kSwigluBlock));
    const v4f_t a = {swiglu_f32(g.x, u.x), swiglu_f32(g.y, u.y), swiglu_f32(g.z, u.z),
                     swiglu_f32(g.w, u.w)};
    store4<BF16>(act, r * Hp + p, a);
    if (SAVE) {
      store4<BF16>(h_saved, gc, g);
      store4<BF16>(h_saved, gc + kSwigluBlock, u);
    }
  }
}

// dgate = da * up * s (1 + g (1 - s)), dup = da * g * s with s = sigmoid(g), float32.
__device__ inline void swiglu_grad(float g, float u, float da, float& dg, float& du) {
  const float s = 1.0f / (1.0f + expf(-g));
  const float gs = g * s;
  dg = da * u * (s + gs * (1.0f - s));
  du = da * gs;
}

template <bool BF16>
__global__ __launch_bounds__(kFfnThreads) void swiglu_backward_kernel(
    const void* __restrict__ h_saved, const float* __restrict__ da, int64_t rows, int Hp,
    void* __restrict__ dh) {
  const int q4 = Hp / 4;
  const int64_t total = rows * q4;
  for (int64_t i = blockIdx.x * int64_t(kFfnThreads) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * kFfnThreads) {
    const int64_t r = i / q4;
    const int p = int(i - r * q4) * 4;
    const int64_t gc = r * 2 * Hp + gate_col(p);
    const v4f_t g = load4<BF16>(h_saved, gc);
    const v4f_t u = load4<BF16>(h_saved, gc + kSwigluBlock);
    const v4f_t d = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(da + r * Hp + p));
    v4f_t dg, du;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float a, b;
      swiglu_grad(g[c], u[c], d[c], a, b);
      dg[c] = a;
      du[c] = b;
    }
    store4<BF16>(dh, gc, dg);
    store4<BF16>(dh, gc + kSwigluBlock, du);
  }
}

inline int ffn_grid(int64_t work) {
  const int64_t blocks = (work + kFfnThreads - 1) / kFfnThreads;
  return int(blocks < 1 ? 1 : (blocks > 16384 ? 16384 : blocks));
}

}  // namespace moonep

using namespace moonep;

extern "C" int moonep_swiglu(const moonep_shape* shape, const float* h, void* act, void* h_saved,
                             void* stream) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (s.Hp % kSwigluBlock) return MOONEP_EINVAL;
  const int64_t rows = int64_t(s.R) * s.S * s.K;
  if (rows == 0) return MOONEP_OK;
  if (!aligned16(h) || !aligned16(act) || (h_saved && !aligned16(h_saved))) return MOONEP_EINVAL;
  const int grid = ffn_grid(rows * (s.Hp / 4));
  hipStream_t strm = as_stream(stream);
  const bool bf = s.dtype == MOONEP_BF16;
  if (bf && h_saved)
    swiglu_kernel<true, true><<<grid, kFfnThreads, 0, strm>>>(h, rows, s.Hp, act, h_saved);
  else if (bf)
    swiglu_kernel<true, false><<<grid, kFfnThreads, 0, strm>>>(h, rows, s.Hp, act, nullptr);
  else if (h_saved)
    swiglu_kernel<false, true><<<grid, kFfnThreads, 0, strm>>>(h, rows, s.Hp, act, h_saved);
  else
    swiglu_kernel<false, false><<<grid, kFfnThreads, 0, strm>>>(h, rows, s.Hp, act, nullptr);
  return launch_status();
}

extern "C" int moonep_swiglu_backward(const moonep_shape* shape, const void* h_saved,
                                      const float* da, void* dh, void* stream) {
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (s.mode != MOONEP_TRAIN) return MOONEP_EMODE;
  if (s.Hp % kSwigluBlock) return MOONEP_EINVAL;
  const int64_t rows = int64_t(s.R) * s.S * s.K;
  if (rows == 0) return MOONEP_OK;
  if (!aligned16(h_saved) || !aligned16(da) || !aligned16(dh)) return MOONEP_EINVAL;
  const int grid = ffn_grid(rows * (s.Hp / 4));
  hipStream_t strm = as_stream(stream);
  if (s.dtype == MOONEP_BF16)
    swiglu_backward_kernel<true><<<grid, kFfnThreads, 0, strm>>>(h_saved, da, rows, s.Hp, dh);
  else
    swiglu_backward_kernel<false><<<grid, kFfnThreads, 0, strm>>>(h_saved, da, rows, s.Hp, dh);
  return launch_status();
}
