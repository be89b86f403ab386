// Host-side entry points shared by every stage: version, status text, shape
// validation, workspace sizing / initialisation and the sticky error word.
#include "common.h"

namespace moonep {

int validate(const moonep_shape* s) {
  if (!s) return MOONEP_EINVAL;
  if (s->R < 1 || s->S < 0 || s->E < 1 || s->K < 1 || s->B < 0) return MOONEP_EINVAL;
  if (s->mode != MOONEP_TRAIN && s->mode != MOONEP_INFER) return MOONEP_EINVAL;
  if (s->dtype != MOONEP_BF16 && s->dtype != MOONEP_FP32) return MOONEP_EINVAL;
  if (s->E % s->R != 0) return MOONEP_EINVAL;
  const int G = s->E / s->R;
  if (s->B > G) return MOONEP_EINVAL;
  // training: B = E/R, so a rank's replicas (all from one remote home group) fit
  if (s->mode == MOONEP_TRAIN && s->B != G) return MOONEP_EINVAL;
  if (s->K > s->E || s->K > 32) return MOONEP_EINVAL;
  // R*S*K < 2^31 without forming a product that can overflow: K <= 32, so R*K fits in
  // 64 bits, and R*K*S >= 2^31 exactly when R*K > floor((2^31 - 1) / S)
  const int64_t rk = int64_t(s->R) * s->K;
  if (s->S > 0 && rk > int64_t(INT32_MAX) / s->S) return MOONEP_EINVAL;
  const int vec = s->dtype == MOONEP_BF16 ? 8 : 4;  // elements per 16-byte vector
  if (s->H < vec || s->Hp < vec || s->H % vec || s->Hp % vec) return MOONEP_EINVAL;
  if (s->E > 1024 || s->R > 1024) return MOONEP_ELIMIT;
  if (int64_t(s->R) * (s->E + s->B + 1) > 8192) return MOONEP_ELIMIT;
  if (int64_t(s->R) * s->B > 4096) return MOONEP_ELIMIT;
  return MOONEP_OK;
}

int elem_bytes(const moonep_shape& s) { return s.dtype == MOONEP_BF16 ? 2 : 4; }

int launch_status() { return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_EHIP; }

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

}  // namespace moonep

using namespace moonep;

extern "C" int moonep_version(void) { return 100; }

extern "C" const char* moonep_strerror(int status) {
  switch (status) {
    case MOONEP_OK: return "ok";
    case MOONEP_EINVAL: return "invalid argument (shape, pointer, alignment or op)";
    case MOONEP_EWORKSPACE: return "workspace too small";
    case MOONEP_EHIP: return "HIP runtime or kernel launch failure";
    case MOONEP_EMODE: return "backward operation on an inference-mode layer";
    case MOONEP_ELIMIT: return "shape beyond a documented size limit";
    default: return "unknown status";
  }
}

extern "C" int moonep_validate_shape(const moonep_shape* shape) { return validate(shape); }

extern "C" size_t moonep_workspace_bytes(const moonep_shape* shape) {
  if (validate(shape) != MOONEP_OK) return 0;
  return ws_layout(*shape).total;
}

extern "C" int moonep_workspace_init(const moonep_shape* shape, void* ws, size_t ws_bytes,
                                     void* stream) {
  int st = validate(shape);
  if (st) return st;
  const WsLayout w = ws_layout(*shape);
  if (!aligned16(ws)) return MOONEP_EINVAL;
  if (ws_bytes < w.total) return MOONEP_EWORKSPACE;
  const size_t n = w.total / 4;
  const int threads = 256;
  const int blocks = int((n + threads - 1) / threads < 4096 ? (n + threads - 1) / threads : 4096);
  fill_u32_kernel<<<blocks, threads, 0, as_stream(stream)>>>(static_cast<uint32_t*>(ws), n, 0u);
  return launch_status();
}

extern "C" int moonep_get_error(const moonep_shape* shape, void* ws, size_t ws_bytes,
                                int32_t* host_flags, int32_t clear) {
  int st = validate(shape);
  if (st) return st;
  const WsLayout w = ws_layout(*shape);
  if (!aligned16(ws) || !host_flags) return MOONEP_EINVAL;
  if (ws_bytes < w.total) return MOONEP_EWORKSPACE;
  if (hipDeviceSynchronize() != hipSuccess) return MOONEP_EHIP;
  int32_t* dflag = ws_ptr<int32_t>(ws, w.flags) + kFlagError;
  if (hipMemcpy(host_flags, dflag, 4, hipMemcpyDeviceToHost) != hipSuccess) return MOONEP_EHIP;
  if (clear) {
    fill_u32_kernel<<<1, 64>>>(reinterpret_cast<uint32_t*>(dflag), 1, 0u);
    if (launch_status()) return MOONEP_EHIP;
    if (hipDeviceSynchronize() != hipSuccess) return MOONEP_EHIP;
  }
  return MOONEP_OK;
}
