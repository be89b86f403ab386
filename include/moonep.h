/*
 * moonep.h -- C ABI of a perfectly balanced expert-parallel MoE layer on AMD
 * Instinct MI355X (gfx950).
 *
 * R expert-parallel ranks are held as R partitions of one GPU's memory; the
 * "symmetric memory" that lets every rank read every other rank's chunk is one
 * device allocation, so no call here talks to another GPU.
 *
 * Sources, cited below by the short name in brackets:
 *   [maestro]  ai-maestro.online, "Moonshot AI open-sources MoonEP, a perfectly
 *              balanced expert parallelism library"
 *   [spaxe]    spaxe.top, "Moonshot AI Open-Sources MoonEP: A Perfectly Balanced
 *              Expert Parallelism Library for MoE Training" (paragraphs, 1-based)
 *   [noticiai] noticiai.com.br, "Moonshot AI libera MoonEP: biblioteca de codigo
 *              aberto para balanceamento perfeito em modelos MoE"
 *
 * Symbols: R ranks, S tokens per rank, E routed experts, G = E/R home experts
 * per rank (rank p owns experts [pG, (p+1)G)), K experts per token, B prefetch
 * slots per rank, H hidden size, Hp = H' the expert intermediate size,
 * SK = S*K the fixed receive count of every rank, N = R*S tokens in all,
 * g = r*S + s the global token id, u = g*K + k the flat (token, k) slot id.
 *
 * Conventions shared by every call:
 *   - All arrays are caller-owned DEVICE memory, row-major, and must be 16-byte
 *     aligned. The library allocates nothing and frees nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *     only enqueue work and return; none synchronises with the host or copies
 *     device to host (except moonep_get_error), so the whole layer can be
 *     captured in a HIP graph. Work is deterministic: no floating-point atomics.
 *   - Arrays typed void* hold the layer dtype (bfloat16 or float32); gates and
 *     every output of expert compute are float32.
 *   - A call returns MOONEP_OK or a negative status before launching anything
 *     when its arguments are invalid (see moonep_strerror).
 *   - A call with nothing to move (S = 0 for dispatch, combine and the SwiGLU
 *     calls; B = 0 for prefetch and reduce_grad) returns MOONEP_OK once the shape
 *     is valid, without reading its pointers, which may then be NULL.
 *   - W_all is the [E+B,H,Hp] expert weight view of every rank at once: one
 *     tensor of E + R*B rows [E+R*B, H, Hp]. Rank q's row i is W_all[i] for
 *     i < E (the home experts, shared by all ranks) and W_all[E + q*B + (i-E)]
 *     for i >= E (q's own prefetch slots) [maestro "The memory contract"].
 */
#ifndef MOONEP_H
#define MOONEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moonep_shape {
  int32_t R, S, E, K, B, H, Hp;
  int32_t mode;   /* MOONEP_TRAIN or MOONEP_INFER */
  int32_t dtype;  /* MOONEP_BF16 or MOONEP_FP32 */
} moonep_shape;

enum {
  MOONEP_OK = 0,
  MOONEP_EINVAL = -1,      /* bad shape, pointer, alignment or op */
  MOONEP_EWORKSPACE = -2,  /* workspace smaller than moonep_workspace_bytes */
  MOONEP_EHIP = -3,        /* a HIP runtime call or kernel launch failed */
  MOONEP_EMODE = -4,       /* backward op requested on an inference layer */
  MOONEP_ELIMIT = -5       /* shape beyond a documented size limit */
};
enum { MOONEP_TRAIN = 0, MOONEP_INFER = 1 };
enum { MOONEP_BF16 = 0, MOONEP_FP32 = 1 };
enum { MOONEP_FWD = 0, MOONEP_DGRAD = 1, MOONEP_WGRAD = 2 };
/* bits of the sticky device error word read by moonep_get_error */
enum { MOONEP_ERR_ID_RANGE = 1, MOONEP_ERR_ID_DUP = 2 };

/* Library version (major*10000 + minor*100 + patch). */
int moonep_version(void);

/* Human-readable text of a status code. Never NULL. */
const char* moonep_strerror(int status);

/*
 * Validate a layer shape. Rules [maestro "The memory contract"; spaxe 7-8]:
 *   R, E >= 1 and E % R == 0; 0 <= B <= E/R; training needs B == E/R (replicas
 *   come from at most one remote home group, so every touched expert is local);
 *   inference allows B < E/R. 1 <= K <= min(E, 32); S >= 0; R*S*K < 2^31;
 *   H, Hp positive multiples of 8 (bf16) or 4 (fp32); mode and dtype one of
 *   their enum values. A shape breaking these gives MOONEP_EINVAL; one that keeps
 *   them but passes a limit below gives MOONEP_ELIMIT.
 * Size limits (MOONEP_ELIMIT): E <= 1024, R <= 1024, R*(E+B+1) <= 8192,
 *   R*B <= 4096.
 */
int moonep_validate_shape(const moonep_shape* shape);

/*
 * Bytes of device workspace that moonep_plan and moonep_grouped_gemm need for
 * `shape` (0 if the shape is invalid). One workspace serves every call of one
 * layer; it also holds the sticky error word. Calls on one workspace must be
 * ordered on one stream (they share it).
 */
size_t moonep_workspace_bytes(const moonep_shape* shape);

/* Zero the workspace (enqueued on `stream`). Required once before first use: besides
 * the sticky error word, the workspace holds a counter that the planner of a small
 * layer (at most 16384 tokens) counts up within a call and sets back to 0 at its end,
 * and a later call relies on finding it at 0. */
int moonep_workspace_init(const moonep_shape* shape, void* ws, size_t ws_bytes, void* stream);

/*
 * Plan the redundant experts for one router output and assign every (token, k)
 * slot its place in its rank's static S*K buffer [maestro "The core idea:
 * dynamic redundant experts", "The memory contract"; noticiai "A ideia central"].
 *
 *   topk_idx       in   int32 [N, K]: expert of slot u = g*K + k; a token names
 *                       an expert at most once
 *   cu_seqlens     out  int32 [R, E+B+1]: rank q's rows of its [E+B] weight view
 *                       hold buffer positions [cu[q][i], cu[q][i+1]);
 *                       cu[q][0] = 0, cu[q][E+B] = S*K
 *   replica_expert out  int32 [R, B]: expert held by q's prefetch slot j, or -1
 *   slot_map       out  int32 [N*K]: slot u -> q*SK + position in q's buffer
 *   src_index      out  int32 [N*K]: inverse of slot_map
 *
 * The rule (the pages fix no planning algorithm, only its invariants):
 *   T_e = slots routed to e, L_p = sum of T_e over p's home experts. Ranks with
 *   L_p > SK donate, ranks with L_p < SK receive, both in ascending id: each
 *   receiver takes all it lacks from the current donor; a donor that runs short
 *   becomes a receiver of the next donor. A donor lays its experts out by
 *   (T_e desc, e asc), hands its receivers consecutive ranges of that layout in
 *   the order it gave them, and keeps the tail. A receiver numbers the distinct
 *   experts of its range j = 0,1,..: j < B takes slot row E+j, j >= B reads the
 *   home row e in place (inference overflow). Slots of one expert are ranked by
 *   u; each row segment holds its slots in ascending u.
 * Outputs are bit-exact and deterministic. Invalid router data (an id outside
 * [0,E): MOONEP_ERR_ID_RANGE; the same id twice in a row: MOONEP_ERR_ID_DUP)
 * sets the sticky error word; an out-of-range id also makes the plan empty
 * (cu_seqlens all 0, replica_expert and slot_map and src_index all -1) so
 * every later call of the layer does nothing out of bounds.
 */
int moonep_plan(const moonep_shape* shape, const int32_t* topk_idx, int32_t* cu_seqlens,
                int32_t* replica_expert, int32_t* slot_map, int32_t* src_index,
                void* ws, size_t ws_bytes, void* stream);

/*
 * Fill every rank's prefetch slots: W_all[E + q*B + j] = W_all[replica_expert[q][j]]
 * for every used slot [maestro "The memory contract": rows [E,E+B) are local
 * prefetch slots filled by buffer.prefetch_weight; "The core idea": duplicated
 * experts are prefetched before expert compute]. Unused slots are not touched.
 *   w_all  in/out  dtype [E + R*B, H, Hp]
 */
int moonep_prefetch_weight(const moonep_shape* shape, const int32_t* replica_expert,
                           void* w_all, void* stream);

/*
 * Fused permute: write each token row straight into its K expert-grouped
 * positions of the ranks' S*K buffers [maestro "The core idea": zero copy,
 * tokens written directly into their expert-grouped positions].
 *   width  H (activations) or Hp (upstream gradients)
 *   src    in   dtype [N, width]
 *   gates  in   NULL, or float32 [N, K]: then row u is scaled by gates[u] in
 *               float32 and rounded once to dtype (round to nearest even for
 *               bfloat16) -- the backward permute of dY
 *   dst    out  dtype [R*SK, width]: dst[slot_map[u]] = (gate *) src[u / K]
 * Slots whose slot_map entry is negative are skipped.
 */
int moonep_dispatch(const moonep_shape* shape, int32_t width, const void* src,
                    const int32_t* slot_map, const float* gates, void* dst, void* stream);

/*
 * Grouped GEMM over the [E+B, H, Hp] view, rows chosen only by cu_seqlens
 * [maestro "The memory contract": the group GEMM addresses experts purely by
 * row index and cu_seqlens selects the active rows]. Empty rows are skipped;
 * nothing is synchronised with the host.
 *   FWD    a = xp  dtype [R*SK, H],  b = w_all, c = out float32 [R*SK, Hp]:
 *          c[rows of (q,i)] = a[rows] @ view_q(i)
 *   DGRAD  a = dyp dtype [R*SK, Hp], b = w_all, c = dxp float32 [R*SK, H]:
 *          c[rows of (q,i)] = a[rows] @ view_q(i)^T
 *   WGRAD  a = xp, b = dyp; for each non-empty (q,i):
 *          D = a[rows]^T @ b[rows] (float32 [H, Hp]);
 *          i <  E: grad_home[i]         += D   (grad_home float32 [E, H, Hp])
 *          i >= E: reduce_buf[q][i - E] += D   (reduce_buf float32 [R, B, H, Hp])
 *          [maestro "The memory contract": fp32 grads mirror the weight layout,
 *          rows [E,E+B) backed by a separate reduce buffer]. WGRAD requires rank
 *          q's rows i < E to be empty unless i is one of q's home experts, as a
 *          training plan leaves them: each grad_home row then has one writer (two
 *          ranks adding into one row would race).
 * Inputs bf16 with float32 accumulation (MFMA), or float32 throughout.
 * Requires H and Hp multiples of 64. DGRAD and WGRAD on an inference layer
 * return MOONEP_EMODE.
 */
int moonep_grouped_gemm(const moonep_shape* shape, int32_t op, const void* a, const void* b,
                        const int32_t* cu_seqlens, float* c, float* grad_home, float* reduce_buf,
                        void* ws, size_t ws_bytes, void* stream);

/* Bytes of the per-device scratch array behind moonep_grouped_gemm_noalloc. */
#define MOONEP_NOALLOC_SCRATCH_BYTES ((size_t)2 << 20)

/*
 * moonep_grouped_gemm for callers that cannot allocate device memory or hold a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments (without the workspace), results and errors
 * as moonep_grouped_gemm, on the same kernels. Its tile lists and tile-queue
 * counters (zeroed by the call's own first kernel) live in a static
 * device array of MOONEP_NOALLOC_SCRATCH_BYTES, one per device, held until the
 * process ends; the call allocates nothing, frees nothing and needs no set-up
 * (the first call on a device resolves the array's address once).
 * Limit: the lists of one call take 256 + align256(16 * (R*(ceil(S*K/64) + E + B)
 * + 1)) + 16 * (R*(E+B) + 1) bytes rounded up to 256 (0.23 MiB at R=8, S=8192,
 * K=8, E=384, B=48); a shape that needs more than the array returns
 * MOONEP_ELIMIT before any launch.
 * Every call on one device shares that device's array, which keeps the last
 * call's lists: calls that can overlap on one device (two streams, two host
 * threads) race and must be ordered by the caller.
 */
int moonep_grouped_gemm_noalloc(const moonep_shape* shape, int32_t op, const void* a,
                                const void* b, const int32_t* cu_seqlens, float* c,
                                float* grad_home, float* reduce_buf, void* stream);

/*
 * Fused unpermute: dst[g] = sum over k ascending of gates[g][k] * src[slot_map[g*K+k]]
 * (gates NULL: weight 1 -- the unpermute of dX), float32 [maestro "The core
 * idea": fused permute/unpermute].
 *   src  in  float32 [R*SK, width];  dst  out  float32 [N, width]
 * Slots whose slot_map entry is negative contribute nothing.
 */
int moonep_combine(const moonep_shape* shape, int32_t width, const float* src,
                   const int32_t* slot_map, const float* gates, float* dst, void* stream);

/*
 * Fold replica gradients home [maestro "The memory contract": reduce_grad reads
 * each rank's own experts' slots from every rank, accumulates into the local
 * parameter grad and zeroes the consumed slots; spaxe 9]:
 *   for q ascending, j ascending with e = replica_expert[q][j] >= 0:
 *     grad_home[e] += reduce_buf[q][j]; reduce_buf[q][j] = 0
 *   reduce_buf  in/out float32 [R, B, H, Hp]; grad_home in/out float32 [E, H, Hp]
 * Unused slots are neither read nor written. Training layers only.
 */
int moonep_reduce_grad(const moonep_shape* shape, const int32_t* replica_expert,
                       float* reduce_buf, float* grad_home, void* stream);

/*
 * ---- Full expert FFN on the same plan --------------------------------------
 * The pages give the weight contract per projection, one [E+B, H, H'] tensor
 * per expert weight, with H' the expert FFN's intermediate size [maestro "The
 * memory contract"]; they do not name the activation. The FFN built from these
 * calls is the gated form
 *     h = x @ W1[e] (gate and up projection),  act = silu(h_gate) * h_up,
 *     z = act @ W2[e] (down projection),        silu(v) = v / (1 + e^-v),
 * on two weight views: W1_all [E+R*B, H, 2H'] and W2_all [E+R*B, H', H], both
 * addressed like W_all and filled by moonep_prefetch_weight with the shapes
 * below. One plan (cu_seqlens, slot_map, replica_expert) and one workspace
 * serve every call of the layer:
 *   up shape    (R,S,E,K,B, H,  2H')  grouped GEMMs of W1, dispatch of x / dy,
 *                                      combine of dX, reduce_grad of dW1
 *   down shape  (R,S,E,K,B, H', H )   grouped GEMMs of W2, combine of z,
 *                                      reduce_grad of dW2
 *   ffn shape   (R,S,E,K,B, H,  H')   the calls below (Hp = H')
 * Gate and up columns of W1 (and of h, h_saved and dh) are interleaved in
 * blocks of MOONEP_SWIGLU_BLOCK: intermediate column p has its gate column at
 * 2*32*(p / 32) + p % 32 and its up column 32 further. Checkpoints in another
 * order are permuted once to this layout.
 */
enum { MOONEP_SWIGLU_BLOCK = 32 };

/*
 * SwiGLU of a gate/up projection computed by moonep_grouped_gemm (FWD, up shape).
 *   h        in   float32 [R*SK, 2*Hp], interleaved gate/up columns
 *   act      out  dtype [R*SK, Hp]: silu(gate) * up in float32, rounded once to
 *                 dtype (round to nearest even for bfloat16)
 *   h_saved  out  NULL, or dtype [R*SK, 2*Hp]: h rounded to dtype, the
 *                 pre-activation the backward pass reads
 * Requires Hp a multiple of 32. Rows of unused buffer positions (none in a
 * valid plan) are processed like any other.
 */
int moonep_swiglu(const moonep_shape* shape, const float* h, void* act, void* h_saved,
                  void* stream);

/*
 * Gate/up grouped GEMM with the SwiGLU in its epilogue: the same values as
 * moonep_grouped_gemm(FWD, up shape) followed by moonep_swiglu, bit for bit,
 * without the float32 h in memory.
 *   xp       in   dtype [R*SK, H]
 *   w1_all   in   dtype [E+R*B, H, 2*Hp] (interleaved gate/up columns)
 *   act      out  dtype [R*SK, Hp];  h_saved  out  NULL or dtype [R*SK, 2*Hp]
 * Requires H a multiple of 64 and Hp a multiple of 32.
 */
int moonep_grouped_gemm_swiglu(const moonep_shape* shape, const void* xp, const void* w1_all,
                               const int32_t* cu_seqlens, void* act, void* h_saved, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * SwiGLU backward: from the saved pre-activation and the gradient of act,
 *   dh_gate = da * up * silu'(gate),  dh_up = da * silu(gate),
 *   silu'(v) = s (1 + v (1 - s)),  s = 1 / (1 + e^-v),
 * in float32, rounded once to dtype.
 *   h_saved  in   dtype [R*SK, 2*Hp];  da  in  float32 [R*SK, Hp]
 *   dh       out  dtype [R*SK, 2*Hp] (interleaved), the operand of the
 *                 backward GEMMs of W1 (DGRAD and WGRAD, up shape)
 * Requires Hp a multiple of 32. Training layers only.
 */
int moonep_swiglu_backward(const moonep_shape* shape, const void* h_saved, const float* da,
                           void* dh, void* stream);

/*
 * ---- Process-global prefetch-slot pool ----------------------------------------
 * The prefetch slots of every layer come from one process-global pool, so the
 * extra memory is R*B expert weights per projection in total, not per layer,
 * while each layer still hands the grouped GEMM one contiguous [E+R*B, H, Hp]
 * tensor [maestro "The memory contract": prefetch slots drawn from a
 * process-global pool shared by all layers; noticiai "O contrato de memória"].
 * A view is one reserved virtual address range: rows [0,E) map the layer's own
 * home-weight allocation (owned by the view), rows [E, E+R*B) map one physical
 * set of the pool. The view's base address is the w_all every other call takes.
 * Views of the same pool set alias the same slot memory: a layer's slots hold
 * its replicas only from its moonep_prefetch_weight until another layer's
 * prefetch on that set; a backward pass prefetches its layer's replicas again.
 *
 * These calls ALLOCATE (device virtual memory) and synchronise where stated;
 * they are set-up calls, not hot-path calls. Home rows start uninitialised.
 * Requires HIP virtual memory support; E*H*Hp*element_size must be a multiple
 * of moonep_vm_granularity() (MOONEP_EINVAL otherwise).
 */
typedef struct moonep_pool moonep_pool;
typedef struct moonep_view moonep_view;

/* Virtual-memory mapping granularity of the current device in bytes, 0 if the
 * device has no virtual memory support. */
size_t moonep_vm_granularity(void);

/* A pool of `nsets` physical slot sets (1..64), each R*B rows of H*Hp elements of
 * shape->dtype, on the current device. B >= 1. */
int moonep_pool_create(const moonep_shape* shape, int32_t nsets, moonep_pool** pool);

/* Physical bytes the pool holds (all sets). */
size_t moonep_pool_bytes(const moonep_pool* pool);

/* Release the pool's physical memory. Destroy every view on it first (releasing a
 * pool whose slots are still mapped is not supported); destroying a view never
 * reads the pool. */
int moonep_pool_destroy(moonep_pool* pool);

/* A layer's [E+R*B, H, Hp] view: fresh home rows plus slot set `set` of `pool`.
 * shape must match the pool's R, B, H, Hp and dtype (E may differ). *w_all
 * receives the view's device address. */
int moonep_view_create(const moonep_shape* shape, moonep_pool* pool, int32_t set,
                       moonep_view** view, void** w_all);

/* Synchronise the device, unmap the view and free its home rows. */
int moonep_view_destroy(moonep_view* view);

/*
 * Read (and if `clear`, reset) the sticky device error word of a workspace.
 * Synchronises the device: for tests and debugging, not for the hot path.
 */
int moonep_get_error(const moonep_shape* shape, void* ws, size_t ws_bytes, int32_t* host_flags,
                     int32_t clear);

#ifdef __cplusplus
}
#endif

#endif /* MOONEP_H */
