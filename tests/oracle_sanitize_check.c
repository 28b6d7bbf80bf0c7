/*
 * Driver for running the CPU oracle (oracle/rope_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host.  Test infrastructure: it calls the oracle's entry
 * points on seeded random configurations of both operations, with every buffer allocated to
 * its exact size (so a read or write one element past a tensor is caught), and checks the
 * status each call returns:
 *   - in-place op: every dtype pair, rank-4 x with a random D, slice (absent, even or odd
 *     start, or empty), B/S/N, broadcast dims of cos/sin, both rotary modes, forward and
 *     gradient, with and without the float64 twin;
 *   - cache op: every dtype, both styles, rope mode and every whitelisted mropeSection with
 *     both cache modes, padded query rows, rotaryDim either side of 16384 (rope mode),
 *     positions in range (status 0) and one out of range (the oracle's out-of-contract
 *     status);
 *   - a few calls that must be refused (NULL data, a bad slice, a bad list).
 * Prints "ok <calls>" or the first failure; exit status 1 on failure.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* Mirror of the oracle's descriptor (the oracle keeps no header). */
typedef struct {
  void *data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} oro_tensor;

int oro_rope_partial_inplace(const oro_tensor *x, const oro_tensor *cos_t, const oro_tensor *sin_t,
                             int64_t rotary_mode, const int64_t *partial_slice,
                             int64_t partial_slice_len, double *x64);
int oro_rope_partial_inplace_backward(const oro_tensor *g, const oro_tensor *cos_t,
                                      const oro_tensor *sin_t, int64_t rotary_mode,
                                      const int64_t *partial_slice, int64_t partial_slice_len,
                                      double *g64);
int oro_rope_with_cos_sin_cache_v2(const oro_tensor *positions, const oro_tensor *query_in,
                                   const oro_tensor *key_in, const oro_tensor *cache,
                                   const int64_t *mrope_section, int64_t mrope_section_len,
                                   int64_t head_size, int is_neox_style, int64_t cache_mode,
                                   const oro_tensor *query_out, const oro_tensor *key_out,
                                   double *q64, double *k64);
const char *oro_last_error(void);

enum { F32 = 0, F16 = 1, BF16 = 2, I64 = 3 };

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t rnd(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545f4914f6cdd1dull;
}
static int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(rnd() % (uint64_t)(hi - lo + 1)); }

static int esize(int dt) { return dt == F32 ? 4 : dt == I64 ? 8 : 2; }

/* A row-major tensor of exactly its size, filled with random finite values. */
static oro_tensor make(int dt, int ndim, const int64_t *shape) {
  oro_tensor t;
  memset(&t, 0, sizeof t);
  t.dtype = dt;
  t.ndim = ndim;
  int64_t n = 1;
  for (int d = ndim - 1; d >= 0; --d) {
    t.shape[d] = shape[d];
    t.stride[d] = n;
    n *= shape[d];
  }
  size_t bytes = (size_t)(n > 0 ? n : 1) * (size_t)esize(dt);
  t.data = malloc(bytes);
  for (int64_t i = 0; i < n; ++i) {
    if (dt == F32) ((float *)t.data)[i] = (float)((int64_t)(rnd() % 2001) - 1000) / 512.0f;
    else if (dt == I64) ((int64_t *)t.data)[i] = 0;
    else ((uint16_t *)t.data)[i] = (uint16_t)(dt == BF16 ? 0x3c00 + rnd() % 0x300 : 0x3000 + rnd() % 0x1000);
  }
  return t;
}

static int64_t numel(const oro_tensor *t) {
  int64_t n = 1;
  for (int d = 0; d < t->ndim; ++d) n *= t->shape[d];
  return n;
}

static int calls = 0, failed = 0;
static void expect(int got, int want, const char *what, int seed) {
  ++calls;
  if (got != want && !failed) {
    failed = 1;
    printf("FAIL %s seed %d: status %d, expected %d (%s)\n", what, seed, got, want,
           oro_last_error());
  }
}

static void inplace_case(int seed) {
  static const int pairs[5][2] = {{F32, F32}, {F16, F16}, {BF16, BF16}, {F16, F32}, {BF16, F32}};
  const int *pr = pairs[pick(0, 4)];
  int64_t D = 2 * pick(1, 40);
  int64_t B = pick(1, 3), S = pick(1, 6), N = pick(1, 4);
  int64_t L = 2 * pick(0, D / 2), start = pick(0, D - L);
  int absent = L == D && start == 0 && pick(0, 1);
  int64_t sl[2] = {start, start + L};
  int64_t xs[4] = {B, S, N, D};
  int64_t cs[4] = {pick(0, 1) ? B : 1, pick(0, 1) ? S : 1, pick(0, 1) ? N : 1, L};
  oro_tensor x = make(pr[0], 4, xs), c = make(pr[1], 4, cs), s = make(pr[1], 4, cs);
  int64_t mode = pick(0, 1);
  double *x64 = pick(0, 1) ? malloc((size_t)numel(&x) * sizeof(double)) : NULL;
  int bwd = (int)pick(0, 1);
  int st = bwd ? oro_rope_partial_inplace_backward(&x, &c, &s, mode, absent ? NULL : sl,
                                                   absent ? 0 : 2, x64)
               : oro_rope_partial_inplace(&x, &c, &s, mode, absent ? NULL : sl, absent ? 0 : 2, x64);
  expect(st, 0, "in-place", seed);
  /* refused calls: a slice past D, NULL data */
  int64_t bad[2] = {start, D + 2};
  expect(oro_rope_partial_inplace(&x, &c, &s, 1, bad, 2, NULL), 161002, "in-place bad slice", seed);
  void *keep = x.data;
  x.data = NULL;
  expect(oro_rope_partial_inplace(&x, &c, &s, 1, NULL, 0, NULL), 161001, "in-place null", seed);
  x.data = keep;
  free(x.data);
  free(c.data);
  free(s.data);
  free(x64);
}

static void cache_case(int seed) {
  static const int64_t lists[5][4] = {{16, 24, 24, 0}, {8, 12, 12, 0}, {24, 20, 20, 0},
                                      {11, 11, 10, 0}, {16, 16, 16, 16}};
  int dt = (int)pick(0, 2);
  int64_t align = 64 / esize(dt);
  int neox = (int)pick(0, 1);
  int kind = (int)pick(0, 5); /* 0: rope, else list kind - 1 */
  const int64_t *sec = kind ? lists[kind - 1] : NULL;
  int64_t nsec = kind == 5 ? 4 : kind ? 3 : 0;
  /* rope mode, 1 in 12: rotaryDim either side of 16384 (the oracle's row buffers are sized
   * per call; every buffer here is allocated to its exact size, so the sanitizer sees any
   * overrun) */
  int long_rd = !kind && pick(0, 11) == 0;
  int64_t rd = kind ? 2 * (sec[0] + sec[1] + sec[2] + sec[3])
                    : long_rd ? align * pick(16384 / align - 2, 24576 / align) : align * pick(1, 4);
  if (rd % align) return; /* [11,11,10] in f32: not a 64-byte multiple */
  int64_t H = rd + align * pick(0, 2);
  int64_t nq = pick(1, 5), nk = pick(1, 3), T = long_rd ? pick(1, 3) : pick(1, 40);
  int64_t max_seq = pick(1, 70);
  int64_t pad = pick(0, 1) * align;
  int64_t cache_mode = nsec == 3 ? pick(0, 1) : 0;
  int64_t qbig_shape[2] = {T, nq * H + pad}, ks[2] = {T, nk * H}, cshape[2] = {max_seq, rd};
  oro_tensor qbig = make(dt, 2, qbig_shape), k = make(dt, 2, ks), cache = make(dt, 2, cshape);
  oro_tensor q = qbig;
  q.shape[1] = nq * H; /* a view of the first nq*H columns: row stride nq*H + pad */
  int64_t qs[2] = {T, nq * H};
  oro_tensor qo = make(dt, 2, qs), ko = make(dt, 2, ks);
  int64_t ps1[1] = {T}, ps2[2] = {nsec, T};
  oro_tensor pos = nsec ? make(I64, 2, ps2) : make(I64, 1, ps1);
  for (int64_t i = 0; i < numel(&pos); ++i) ((int64_t *)pos.data)[i] = pick(0, max_seq - 1);
  double *q64 = malloc((size_t)(T * nq * H) * sizeof(double));
  double *k64 = malloc((size_t)(T * nk * H) * sizeof(double));
  int st = oro_rope_with_cos_sin_cache_v2(&pos, &q, &k, &cache, sec, nsec, H, neox, cache_mode,
                                          &qo, &ko, pick(0, 1) ? q64 : NULL, k64);
  expect(st, 0, "cache", seed);
  ((int64_t *)pos.data)[numel(&pos) - 1] = max_seq; /* outside the cache: out of contract */
  expect(oro_rope_with_cos_sin_cache_v2(&pos, &q, &k, &cache, sec, nsec, H, neox, cache_mode,
                                        &qo, &ko, NULL, NULL), -1, "cache position", seed);
  int64_t wrong[3] = {16, 24, 23};
  expect(oro_rope_with_cos_sin_cache_v2(&pos, &q, &k, &cache, wrong, 3, H, neox, 0, &qo, &ko,
                                        NULL, NULL), 161002, "cache bad list", seed);
  free(qbig.data);
  free(k.data);
  free(cache.data);
  free(qo.data);
  free(ko.data);
  free(pos.data);
  free(q64);
  free(k64);
}

int main(void) {
  for (int seed = 0; seed < 3000 && !failed; ++seed) inplace_case(seed);
  for (int seed = 0; seed < 1500 && !failed; ++seed) cache_case(seed);
  if (failed) return 1;
  printf("ok %d\n", calls);
  return 0;
}
