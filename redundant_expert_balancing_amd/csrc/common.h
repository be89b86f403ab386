// Internal definitions shared by the HIP sources of the moonep library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moonep.h"

namespace moonep {

// Router tokens per planning chunk: one 64-wide wavefront owns a chunk, one lane
// per token while counting, 64 consecutive slots per step while assigning.
constexpr int kChunkTokens = 64;
// Chunks per partition of the planner's column scan (16 wavefronts x 4 chunks).
constexpr int kScanPart = 64;
// Layers of at most kFusedMaxChunks chunks count, scan and solve in one launch:
// kFusedChunks chunks (one per wavefront) per workgroup, each workgroup a partition.
constexpr int kFusedChunks = 16;
constexpr int kFusedMaxChunks = 256;
// Smallest GEMM M tile; sizes the tile list in the workspace.
constexpr int kMinTileM = 64;

// Sticky error word and per-call words at the head of the workspace.
enum FlagWord {
  kFlagError = 0, kFlagPlanValid = 1, kFlagTileCount = 2, kFlagTileCountTail = 3,
  kFlagPlanArrive = 4,   // workgroups of the fused planner done counting (back to 0 after)
  kFlagQueue = 16,   // 2 x kQueueWords GEMM tile-queue counters
  kFlagWords = 64
};
constexpr int kQueueWords = 8;   // one tile-queue counter per XCD

struct WsLayout {
  size_t flags, part, counts, piece_ptr, piece_tlo, piece_base, tiles, tiles_tail, total;
  int64_t nchunk, npart, nfused, max_pieces, max_tiles, max_tail;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(const moonep_shape& s) {
  WsLayout w{};
  const int64_t N = int64_t(s.R) * s.S;
  const int64_t SK = int64_t(s.S) * s.K;
  w.nchunk = (N + kChunkTokens - 1) / kChunkTokens;
  w.npart = (w.nchunk + kScanPart - 1) / kScanPart;
  w.nfused = w.nchunk > 0 && w.nchunk <= kFusedMaxChunks
                 ? (w.nchunk + kFusedChunks - 1) / kFusedChunks : 0;
  w.max_pieces = int64_t(s.E) + 2 * int64_t(s.R) + 8;
  w.max_tiles = int64_t(s.R) * ((SK + kMinTileM - 1) / kMinTileM + s.E + s.B) + 1;
  w.max_tail = int64_t(s.R) * (s.E + s.B) + 1;   // at most one short tail per segment
  size_t o = 0;
  w.flags = o;      o = align256(o + kFlagWords * 4);
  w.part = o;       o = align256(o + size_t(w.npart > w.nfused ? w.npart : w.nfused) * s.E * 4);
  w.counts = o;     o = align256(o + size_t(w.nchunk) * s.E * 4);
  w.piece_ptr = o;  o = align256(o + size_t(s.E + 1) * 4);
  w.piece_tlo = o;  o = align256(o + size_t(w.max_pieces) * 4);
  w.piece_base = o; o = align256(o + size_t(w.max_pieces) * 4);
  w.tiles = o;      o = align256(o + size_t(w.max_tiles) * 16);
  w.tiles_tail = o; o = align256(o + size_t(w.max_tail) * 16);
  w.total = o;
  return w;
}

template <typename T>
inline T* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

inline bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// float32 -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__device__ inline uint32_t bf16_rne_bits(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

// SwiGLU in float32: silu(g) * u with silu(g) = g / (1 + e^-g). Every kernel that
// produces the activation calls this one function, so all of them agree bit for bit.
__device__ inline float swiglu_f32(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Gate/up columns of the FFN's first projection are interleaved in blocks of
// kSwigluBlock: intermediate column p has its gate at 2*kSwigluBlock*(p / kSwigluBlock)
// + p % kSwigluBlock and its up projection kSwigluBlock further.
constexpr int kSwigluBlock = MOONEP_SWIGLU_BLOCK;

// Host-side validation shared by all entry points (defined in api.hip).
int validate(const moonep_shape* s);
int elem_bytes(const moonep_shape& s);
int launch_status();  // MOONEP_OK or MOONEP_EHIP after the last launch

}  // namespace moonep
