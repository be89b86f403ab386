/* Host arithmetic of include/moonep.h under extreme and random shapes, for a build
 * with host-side sanitizers: shape validation against the rules the header states
 * (restated here in 128-bit arithmetic), workspace sizing (zero exactly for an
 * invalid shape, a multiple of 256 otherwise), status text for every code, and every
 * entry point given NULL device pointers, which must be refused on the host. Exit 0
 * when every check passes; prints the first failing checks otherwise. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moonep.h"

static int fails = 0;
static void fail(const char* what, const moonep_shape* s, int got, int want) {
  if (++fails <= 10)
    fprintf(stderr, "check failed: %s: R=%d S=%d E=%d K=%d B=%d H=%d Hp=%d mode=%d dtype=%d got %d want %d\n",
            what, s->R, s->S, s->E, s->K, s->B, s->H, s->Hp, s->mode, s->dtype, got, want);
}

/* xorshift64 (Marsaglia, "Xorshift RNGs", J. Stat. Softw. 8(14), 2003) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}

static const int special[] = {INT_MIN, -65536, -1, 0, 1, 2, 3, 4, 7, 8, 12, 16, 31, 32, 33,
                              48, 64, 384, 1023, 1024, 1025, 2048, 4096, 7168, 8192, 8193,
                              65536, 1 << 20, 1 << 30, INT_MAX - 1, INT_MAX};
#define NSPECIAL ((int)(sizeof special / sizeof *special))

static int pick(void) {
  const uint64_t r = next_u64();
  switch (r % 3) {
    case 0: return special[(r >> 8) % NSPECIAL];
    case 1: return (int)((r >> 8) % 4097);
    default: return (int)(uint32_t)(r >> 16);
  }
}

/* The status the header's rules give: shape rules first (MOONEP_EINVAL), then the
 * size limits (MOONEP_ELIMIT). */
static int expected_status(const moonep_shape* s) {
  if (s->R < 1 || s->E < 1 || s->K < 1 || s->S < 0 || s->B < 0) return MOONEP_EINVAL;
  if (s->mode != MOONEP_TRAIN && s->mode != MOONEP_INFER) return MOONEP_EINVAL;
  if (s->dtype != MOONEP_BF16 && s->dtype != MOONEP_FP32) return MOONEP_EINVAL;
  if (s->E % s->R != 0) return MOONEP_EINVAL;
  const int G = s->E / s->R;
  if (s->B > G || (s->mode == MOONEP_TRAIN && s->B != G)) return MOONEP_EINVAL;
  if (s->K > s->E || s->K > 32) return MOONEP_EINVAL;
  if ((__int128)s->R * s->S * s->K >= ((__int128)1 << 31)) return MOONEP_EINVAL;
  const int vec = s->dtype == MOONEP_BF16 ? 8 : 4;
  if (s->H < vec || s->Hp < vec || s->H % vec || s->Hp % vec) return MOONEP_EINVAL;
  if (s->E > 1024 || s->R > 1024) return MOONEP_ELIMIT;
  if ((__int128)s->R * ((__int128)s->E + s->B + 1) > 8192) return MOONEP_ELIMIT;
  if ((__int128)s->R * s->B > 4096) return MOONEP_ELIMIT;
  return MOONEP_OK;
}

static void check_shape(const moonep_shape* s) {
  const int want = expected_status(s);
  const int st = moonep_validate_shape(s);
  if (st != want) fail("validate", s, st, want);
  const size_t ws = moonep_workspace_bytes(s);
  if ((ws == 0) != (st != MOONEP_OK) || ws % 256) fail("workspace bytes", s, (int)(ws != 0), st == MOONEP_OK);
  /* NULL device pointers: refused on the host (MOONEP_EHIP would mean a device call
   * was made), except that a valid call with nothing to move returns MOONEP_OK */
  const int no_tokens = st == MOONEP_OK && s->S == 0;
  const int no_slots = st == MOONEP_OK && s->B == 0;
  /* the SwiGLU calls also need Hp in whole gate/up column blocks */
  const int swiglu_empty = no_tokens && s->Hp % MOONEP_SWIGLU_BLOCK == 0;
  const int train = s->mode == MOONEP_TRAIN;
  const int empty[] = {0, no_slots, no_tokens, 0, 0, 0, no_tokens, no_slots && train,
                       swiglu_empty, 0, swiglu_empty && train, 0, 0, 0};
  const int calls[] = {
      moonep_plan(s, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL),
      moonep_prefetch_weight(s, NULL, NULL, NULL),
      moonep_dispatch(s, s->H, NULL, NULL, NULL, NULL, NULL),
      moonep_grouped_gemm(s, MOONEP_FWD, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL),
      moonep_grouped_gemm(s, MOONEP_WGRAD, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL),
      moonep_grouped_gemm_noalloc(s, MOONEP_DGRAD, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
      moonep_combine(s, s->Hp, NULL, NULL, NULL, NULL, NULL),
      moonep_reduce_grad(s, NULL, NULL, NULL, NULL),
      moonep_swiglu(s, NULL, NULL, NULL, NULL),
      moonep_grouped_gemm_swiglu(s, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL),
      moonep_swiglu_backward(s, NULL, NULL, NULL, NULL),
      moonep_workspace_init(s, NULL, 0, NULL),
      moonep_get_error(s, NULL, 0, NULL, 0),
      moonep_view_create(s, NULL, 0, NULL, NULL),
  };
  for (int i = 0; i < (int)(sizeof calls / sizeof *calls); ++i) {
    if (calls[i] == MOONEP_EHIP || (calls[i] == MOONEP_OK) != empty[i])
      fail("NULL pointers refused unless the call is empty", s, calls[i], i);
  }
  if (st != MOONEP_OK) {
    moonep_pool* pool = NULL;
    const int pc = moonep_pool_create(s, 1, &pool);
    if (pc != st || pool != NULL) fail("pool_create on an invalid shape", s, pc, st);
  }
}

int main(void) {
  /* status text: never NULL, never empty */
  for (int c = -100; c <= 100; ++c) {
    const char* t = moonep_strerror(c);
    if (!t || !*t) { fprintf(stderr, "check failed: strerror(%d)\n", c); ++fails; }
  }
  if (moonep_validate_shape(NULL) != MOONEP_EINVAL || moonep_workspace_bytes(NULL) != 0) {
    fprintf(stderr, "check failed: NULL shape\n");
    ++fails;
  }
  /* edge shapes: the largest products the rules admit before the size limits */
  const moonep_shape edges[] = {
      {INT_MAX, INT_MAX, INT_MAX, 32, 1, 8, 8, MOONEP_TRAIN, MOONEP_BF16},
      {INT_MAX, INT_MAX, INT_MAX, 32, 0, 8, 8, MOONEP_INFER, MOONEP_FP32},
      {1, INT_MAX, INT_MAX, 32, INT_MAX, 8, 8, MOONEP_TRAIN, MOONEP_BF16},
      {1024, 65536, 1024, 32, 1, 8, 8, MOONEP_TRAIN, MOONEP_BF16},
      {1, (1 << 26) - 1, 32, 32, 32, 8, 8, MOONEP_TRAIN, MOONEP_BF16},
      {1, 1 << 26, 32, 32, 32, 8, 8, MOONEP_TRAIN, MOONEP_BF16},
      {8, 8192, 384, 8, 48, INT_MAX - 7, INT_MAX - 7, MOONEP_TRAIN, MOONEP_BF16},
      {8, 0, 384, 8, 48, 7168, 2048, MOONEP_TRAIN, MOONEP_BF16},
      {1024, 0, 1024, 1, 1, 4, 4, MOONEP_TRAIN, MOONEP_FP32},
      {8, 8, 8, 1, 1, 8, 8, 2, MOONEP_BF16},
      {8, 8, 8, 1, 1, 8, 8, MOONEP_TRAIN, -1},
  };
  for (int i = 0; i < (int)(sizeof edges / sizeof *edges); ++i) check_shape(&edges[i]);
  /* random shapes: either seven independent draws, or a valid shape with one field
   * replaced by a draw */
  for (int it = 0; it < 200000; ++it) {
    moonep_shape s;
    if (next_u64() & 1) {
      s.R = pick(); s.S = pick(); s.E = pick(); s.K = pick(); s.B = pick();
      s.H = pick(); s.Hp = pick();
      s.mode = (int)(next_u64() % 4) - 1;
      s.dtype = (int)(next_u64() % 4) - 1;
    } else {
      const int R = 1 << (next_u64() % 11), G = 1 + (int)(next_u64() % 64);
      s.R = R; s.E = R * G; s.mode = (int)(next_u64() & 1);
      s.B = s.mode == MOONEP_TRAIN ? G : (int)(next_u64() % (G + 1));
      s.K = 1 + (int)(next_u64() % (s.E < 32 ? s.E : 32));
      s.S = (int)(next_u64() % 100000);
      s.dtype = (int)(next_u64() & 1);
      s.H = 8 * (1 + (int)(next_u64() % 1024)); s.Hp = 8 * (1 + (int)(next_u64() % 1024));
      int* f[] = {&s.R, &s.S, &s.E, &s.K, &s.B, &s.H, &s.Hp};
      *f[next_u64() % 7] = pick();
    }
    check_shape(&s);
  }
  if (fails == 0) printf("abi_fuzz: all checks passed\n");
  return fails ? 1 : 0;
}
