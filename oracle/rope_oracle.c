/*
 * rope_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU definition of the two RoPE operations, used to check the GPU
 * library and nothing else.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark load it; the product path never does.  It shares no source, header,
 * helper or table with the GPU library: the descriptor type, the dtype decoding, the
 * rounding routines and the validation below are all written here on their own.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no -ffast-math, IEEE denormals kept), so
 * every float operation below is one IEEE binary32 operation rounded to nearest-even.
 *
 * Pages cited (the reader has the pages; titles are given once here):
 *   [IPRM]  "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码
 *            接口详解与实现剖析"
 *   [RSCC]  "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的
 *            计算原理与 aclnn 两段式调用实战"
 *
 * Arithmetic precision.  [IPRM §返回值与错误码] says a half-precision x may take FLOAT32 cos/sin,
 * which are then raised to FLOAT32 for the computation; the oracle therefore upcasts every
 * operand to binary32, evaluates each product and each sum as written in the formulas (one
 * rounding each, no fused multiply-add) and rounds once to the tensor dtype at the store.
 * Every compute entry point also fills an optional binary64 "twin" (same loops, double
 * arithmetic, no final rounding) that the tests use for error analysis.
 *
 * Readings of points the pages leave open (each one is listed in the design notes):
 *  R1 interleave rotation: x_rotate[2i] = -x[2i+1], x_rotate[2i+1] = x[2i] (pairs counted
 *     from the slice start), i.e. the negate-and-swap is interleaved per pair;
 *  R2 partial_slice absent -> [0, D); an explicit [s, s] -> no-op;
 *  R3 the no-op returns before the cos/sin last-dim check;
 *  R5 cos/sin are per element: cos[j] multiplies element j of the slice;
 *  R6 each of the B, S, N dims of cos/sin is either 1 (broadcast) or equal to x's;
 *  R8 GPT-J stack((o1, o2), -1) is flattened, i.e. o1/o2 interleave;
 *  R9 mropeSection[0] > 0 selects mrope; the whitelist is the five lists of [RSCC §入参校验逻辑];
 *  R11 a position outside [0, maxSeqLen) is outside the contract: the oracle refuses it;
 *  R12 an in-place call on an empty x is a successful no-op; the cache op requires non-empty
 *      inputs ([RSCC §入参校验逻辑]);
 *  R18 interleaved stitching (cacheMode 1) takes the printed bound 3*mropeSection[1] for rows
 *      1 and 2;
 *  R20 the in-place gradient is the transpose of the forward map (the page gives no formula);
 *  R21 rotary_mode 0 (half mode, listed but not enabled on the pages) is enabled: x1 and x2
 *      are the first and second halves of the slice, x_rotate = cat(-x2, x1), the same formula
 *      x*cos + x_rotate*sin; 2 and 3 stay invalid.
 *  R22 the in-place op writes xRef while reading cos and sin, so xRef may share no memory
 *      with either (161002); cos and sin are only read and may share memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* Status values printed in [IPRM §返回值与错误码] (error-code table). */
#define ORO_OK 0
#define ORO_ERR_PARAM_NULLPTR 161001
#define ORO_ERR_PARAM_INVALID 161002
/* Oracle-only: the call is outside the contract (a position outside the cache). */
#define ORO_ERR_OUTSIDE_CONTRACT (-1)
/* Oracle-only: the host could not give the oracle its per-call row buffers. */
#define ORO_ERR_OUT_OF_MEMORY (-2)

/* dtype codes of the descriptor (the same numbering as the library's interface, since the
 * harness hands the same descriptions to both). */
enum { ORO_F32 = 0, ORO_F16 = 1, ORO_BF16 = 2, ORO_I64 = 3 };

typedef struct {
  void *data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4]; /* in elements */
} oro_tensor;

static char g_err[512];

static int fail(int code, const char *msg) {
  snprintf(g_err, sizeof g_err, "%s", msg);
  return code;
}

const char *oro_last_error(void) { return g_err; }

/* ------------------------------------------------------------------------------------------
 * binary16 / bfloat16 <-> binary32, written from the IEEE 754 encodings.
 * ------------------------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* bfloat16 keeps the upper 16 bits of a binary32: decoding is exact. */
float oro_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float oro_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  float v;
  if (e == 0)
    v = ldexpf((float)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = (m == 0) ? INFINITY : NAN;
  else
    v = ldexpf((float)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* Round-to-nearest-even of a binary32 to bfloat16: keep the upper half, look at the 16
 * dropped bits; above half -> up, exactly half -> up only if the kept part is odd. */
uint16_t oro_round_bf16(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN: keep the sign, return a quiet NaN */
    return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
  uint32_t kept = u >> 16;
  uint32_t dropped = u & 0xffffu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u; /* carries into exp */
  return (uint16_t)kept;
}

/* Round-to-nearest-even of a binary32 to binary16.  For |v| with binary exponent E the
 * binary16 quantum is 2^(max(E,-14)-10); k = RNE(|v| / quantum) is the integer significand
 * (k in [0, 2048]); the encoding is ((max(E,-14)+15) << 10) + k - 1024, which also covers
 * subnormals (E < -14) and the carry k == 2048; anything at or above 0x7c00 is infinity. */
uint16_t oro_round_f16(float f) {
  uint32_t u = f32_bits(f);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t e = (u >> 23) & 0xffu;
  uint32_t m = u & 0x7fffffu;
  if (e == 0xffu) return (uint16_t)(sign | (m ? 0x7e00u : 0x7c00u)); /* NaN / inf */
  if (e == 0 && m == 0) return sign;                                  /* signed zero */
  /* |v| = sig * 2^(ee - 150), sig < 2^24 */
  uint32_t sig = (e == 0) ? m : (m | 0x800000u);
  int ee = (e == 0) ? 1 : (int)e;
  int E = ee - 127; /* exponent of the leading bit for normal inputs */
  if (e == 0) E = -127; /* binary32 subnormals are far below the binary16 range */
  int Ec = E < -14 ? -14 : E;
  int qe = Ec - 10;                 /* quantum exponent */
  int shift = qe - (ee - 150);      /* k = sig / 2^shift, rounded */
  uint32_t k;
  if (shift <= 0) {
    k = sig << (-shift); /* cannot happen for finite binary16 range but keep it exact */
  } else if (shift >= 32) {
    k = 0;
  } else {
    uint64_t s64 = sig;
    uint64_t q = s64 >> shift;
    uint64_t rem = s64 - (q << shift);
    uint64_t half = (uint64_t)1 << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1;
    k = (uint32_t)q;
  }
  int64_t enc = ((int64_t)(Ec + 15) << 10) + (int64_t)k - 1024;
  if (enc >= 0x7c00) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)enc);
}

/* Array forms, used by the exhaustive tests of the rounding routines. */
void oro_round_bf16_array(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oro_round_bf16(in[i]);
}
void oro_round_f16_array(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oro_round_f16(in[i]);
}
void oro_f16_to_f32_array(const uint16_t *in, float *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oro_f16_to_f32(in[i]);
}

/* ------------------------------------------------------------------------------------------
 * Element access through a descriptor.
 * ------------------------------------------------------------------------------------------ */

static int elem_size(int dtype) {
  switch (dtype) {
    case ORO_F32: return 4;
    case ORO_F16: return 2;
    case ORO_BF16: return 2;
    case ORO_I64: return 8;
    default: return 0;
  }
}

/* Exact upcast of element `off` (in elements from data) to binary32. */
static float load_f32(const oro_tensor *t, int64_t off) {
  const char *p = (const char *)t->data;
  if (t->dtype == ORO_F32) {
    float v;
    memcpy(&v, p + off * 4, 4);
    return v;
  }
  uint16_t h;
  memcpy(&h, p + off * 2, 2);
  return t->dtype == ORO_F16 ? oro_f16_to_f32(h) : oro_bf16_to_f32(h);
}

/* One rounding of a binary32 result to the tensor dtype, then the store. */
static void store_rounded(const oro_tensor *t, int64_t off, float v) {
  char *p = (char *)t->data;
  if (t->dtype == ORO_F32) {
    memcpy(p + off * 4, &v, 4);
    return;
  }
  uint16_t h = t->dtype == ORO_F16 ? oro_round_f16(v) : oro_round_bf16(v);
  memcpy(p + off * 2, &h, 2);
}

/* Raw bit copy of one element (pass-through data is never converted). */
static void copy_bits(const oro_tensor *dst, int64_t doff, const oro_tensor *src, int64_t soff) {
  int es = elem_size(src->dtype);
  memcpy((char *)dst->data + doff * es, (const char *)src->data + soff * es, (size_t)es);
}

static int64_t load_i64(const oro_tensor *t, int64_t off) {
  int64_t v;
  memcpy(&v, (const char *)t->data + off * 8, 8);
  return v;
}

static int shape_ok(const oro_tensor *t) {
  if (t->ndim < 1 || t->ndim > 4) return 0;
  for (int d = 0; d < t->ndim; ++d)
    if (t->shape[d] < 0) return 0;
  return 1;
}

/* Element count; INT64_MAX when the product of the dims would not fit. */
static int64_t numel(const oro_tensor *t) {
  int64_t n = 1;
  for (int d = 0; d < t->ndim; ++d) {
    if (t->shape[d] != 0 && n > INT64_MAX / t->shape[d]) return INT64_MAX;
    n *= t->shape[d];
  }
  return n;
}

/* A descriptor no real buffer can have: more than 2^53 elements, or its furthest element
 * 2^53 or more elements from the first (sum over dims of (size - 1) * |stride|).  Such a
 * tensor is an invalid argument (161002, [IPRM §返回值与错误码]); rejecting it also keeps
 * every index computed below inside int64. */
static int beyond_limits(const oro_tensor *t) {
  const int64_t lim = (int64_t)1 << 53;
  int64_t n = 1, reach = 0;
  for (int d = 0; d < t->ndim; ++d) {
    const int64_t size = t->shape[d], stride = t->stride[d];
    if (size != 0 && n > lim / size) return 1;
    n *= size;
    if (size < 2) continue;
    if (stride == INT64_MIN) return 1;
    const int64_t step = stride < 0 ? -stride : stride;
    if (step != 0 && size - 1 > (lim - 1 - reach) / step) return 1;
    reach += (size - 1) * step;
  }
  return 0;
}

/* Row-major contiguity; the stride of a dimension of size 1 does not matter, and a tensor
 * with no elements has no layout to check (reading R12: an empty xRef is a no-op). */
static int contiguous(const oro_tensor *t) {
  if (numel(t) == 0) return 1;
  int64_t expect = 1;
  for (int d = t->ndim - 1; d >= 0; --d) {
    if (t->shape[d] != 1 && t->stride[d] != expect) return 0;
    expect *= t->shape[d];
  }
  return 1;
}

static int is_float_dtype(int dt) { return dt == ORO_F32 || dt == ORO_F16 || dt == ORO_BF16; }

/* Whether two contiguous tensors share any byte. */
static int contiguous_spans_meet(const oro_tensor *a, const oro_tensor *b) {
  const uintptr_t a0 = (uintptr_t)a->data, b0 = (uintptr_t)b->data;
  const uintptr_t a1 = a0 + (uintptr_t)numel(a) * (uintptr_t)elem_size(a->dtype);
  const uintptr_t b1 = b0 + (uintptr_t)numel(b) * (uintptr_t)elem_size(b->dtype);
  return a0 < b1 && b0 < a1;
}

/* ==========================================================================================
 * Operation A: in-place partial RoPE, interleave mode (and half mode, reading R21).
 *   [IPRM §计算原理与公式]     x1 = x[..., ::2], x2 = x[..., 1::2], x_rotate from -x2 and x1,
 *                              x = x*cos + x_rotate*sin (reading R1: per-pair interleave);
 *   [IPRM §参数说明]           rotary_mode 0 is half mode, 1 interleave;
 *   [IPRM §partial_slice 局部旋转机制] only x[..., start:end) is rotated, cos/sin cover that slice;
 *   [IPRM §约束说明]           D <= 1024, D even, slice length even, cos/sin last dim == slice
 *                              length, cos/sin broadcast to BSND, contiguous tensors only;
 *   [IPRM §返回值与错误码]     161001 for null tensors, 161002 for every other invalid input.
 * ========================================================================================== */
/* Half mode on one row's slice (reading R21): with h = L/2, x1 = slice[0:h], x2 = slice[h:L],
 *   x_rotate = cat(-x2, x1), i.e. x_rotate[i] = -slice[i+h] for i < h and slice[i-h] above;
 *   forward   y = slice*cos + x_rotate*sin;
 *   gradient  the map is y = C x + S R x (C, S diagonal, R the rotate-half matrix), so
 *             dx = C g + R^T S g with (R^T v)[i] = v[i+h] for i < h and -v[i-h] above.
 * The whole slice is read before any element is written (the op is in place). */
static void half_mode_row(const oro_tensor *x, const oro_tensor *cos_t, const oro_tensor *sin_t,
                          int64_t xs, int64_t crow, int64_t L, double *x64, int backward) {
  float v[1024]; /* L <= D <= 1024 */
  const int64_t h = L / 2;
  for (int64_t i = 0; i < L; ++i) v[i] = load_f32(x, xs + i);
  for (int64_t i = 0; i < L; ++i) {
    const float c = load_f32(cos_t, crow + i), sn = load_f32(sin_t, crow + i);
    float p = v[i] * c, q;
    double q64;
    if (!backward) {
      const float rot = i < h ? -v[i + h] : v[i - h];
      q = rot * sn;
      q64 = (double)rot * (double)sn;
    } else if (i < h) {
      const float sp = load_f32(sin_t, crow + i + h);
      q = v[i + h] * sp;
      q64 = (double)v[i + h] * (double)sp;
    } else {
      const float sp = load_f32(sin_t, crow + i - h);
      q = -(v[i - h] * sp);
      q64 = -((double)v[i - h] * (double)sp);
    }
    store_rounded(x, xs + i, p + q);
    if (x64) x64[xs + i] = (double)v[i] * (double)c + q64;
  }
}

static int partial_inplace(const oro_tensor *x, const oro_tensor *cos_t, const oro_tensor *sin_t,
                           int64_t rotary_mode, const int64_t *partial_slice,
                           int64_t partial_slice_len, double *x64, int backward) {
  /* null checks */
  if (!x || !cos_t || !sin_t) return fail(ORO_ERR_PARAM_NULLPTR, "xRef, cos or sin is null");
  if (!partial_slice && partial_slice_len > 0)
    return fail(ORO_ERR_PARAM_NULLPTR, "partialSlice is null but its length is not 0");
  const oro_tensor *ts[3] = {x, cos_t, sin_t};
  for (int i = 0; i < 3; ++i)
    if (shape_ok(ts[i]) && numel(ts[i]) > 0 && !ts[i]->data)
      return fail(ORO_ERR_PARAM_NULLPTR, "a non-empty tensor has a null data pointer");

  /* dtypes: x in {f32, f16, bf16}; cos, sin equal; cos in {x dtype, f32} */
  if (!is_float_dtype(x->dtype)) return fail(ORO_ERR_PARAM_INVALID, "xRef dtype unsupported");
  if (cos_t->dtype != sin_t->dtype) return fail(ORO_ERR_PARAM_INVALID, "cos and sin dtypes differ");
  if (!(cos_t->dtype == x->dtype || cos_t->dtype == ORO_F32))
    return fail(ORO_ERR_PARAM_INVALID, "cos/sin dtype must equal xRef's or be float32");

  if (rotary_mode != 0 && rotary_mode != 1)
    return fail(ORO_ERR_PARAM_INVALID, "rotary_mode must be 1 (interleave) or 0 (half)");

  /* shapes */
  for (int i = 0; i < 3; ++i)
    if (!shape_ok(ts[i]) || ts[i]->ndim != 4)
      return fail(ORO_ERR_PARAM_INVALID, "xRef, cos and sin must be 4-D");
  for (int i = 0; i < 3; ++i)
    if (beyond_limits(ts[i])) return fail(ORO_ERR_PARAM_INVALID, "tensor too large to exist");
  for (int d = 0; d < 4; ++d)
    if (cos_t->shape[d] != sin_t->shape[d])
      return fail(ORO_ERR_PARAM_INVALID, "cos and sin shapes differ");
  const int64_t B = x->shape[0], S = x->shape[1], N = x->shape[2], D = x->shape[3];
  if (D > 1024) return fail(ORO_ERR_PARAM_INVALID, "last dim of xRef exceeds 1024");
  if (D % 2 != 0) return fail(ORO_ERR_PARAM_INVALID, "last dim of xRef is odd");

  /* slice (reading R2) */
  int64_t start = 0, end = D;
  if (partial_slice_len != 0 || partial_slice) {
    if (partial_slice_len != 2) return fail(ORO_ERR_PARAM_INVALID, "partialSlice length must be 2");
    start = partial_slice[0];
    end = partial_slice[1];
  }
  if (start < 0 || end < 0 || end > D || end - start < 0)
    return fail(ORO_ERR_PARAM_INVALID, "partialSlice out of range");
  const int64_t L = end - start;
  if (L % 2 != 0) return fail(ORO_ERR_PARAM_INVALID, "partialSlice length is odd");

  if (!contiguous(x) || !contiguous(cos_t) || !contiguous(sin_t))
    return fail(ORO_ERR_PARAM_INVALID, "non-contiguous tensors are not supported");

  /* reading R3: the empty slice returns before the cos/sin last-dim check */
  if (L == 0) {
    if (x64)
      for (int64_t i = 0; i < numel(x); ++i) x64[i] = (double)load_f32(x, i);
    return ORO_OK;
  }

  if (cos_t->shape[3] != L)
    return fail(ORO_ERR_PARAM_INVALID, "cos/sin last dim must equal the slice length");
  for (int d = 0; d < 3; ++d)
    if (!(cos_t->shape[d] == 1 || cos_t->shape[d] == x->shape[d]))
      return fail(ORO_ERR_PARAM_INVALID, "cos/sin do not broadcast to xRef");
  /* reading R22: xRef is written in place, so it may share no memory with cos or sin (they
   * are only read, and may share memory with each other) */
  if (numel(x) > 0 && (contiguous_spans_meet(x, cos_t) || contiguous_spans_meet(x, sin_t)))
    return fail(ORO_ERR_PARAM_INVALID, "xRef overlaps cos or sin");

  /* fp64 twin of untouched data: exact copies */
  if (x64)
    for (int64_t i = 0; i < numel(x); ++i) x64[i] = (double)load_f32(x, i);

  for (int64_t b = 0; b < B; ++b)
    for (int64_t s = 0; s < S; ++s)
      for (int64_t n = 0; n < N; ++n) {
        int64_t xrow = ((b * S + s) * N + n) * D;
        int64_t bc = cos_t->shape[0] == 1 ? 0 : b;
        int64_t sc = cos_t->shape[1] == 1 ? 0 : s;
        int64_t nc = cos_t->shape[2] == 1 ? 0 : n;
        int64_t crow = ((bc * cos_t->shape[1] + sc) * cos_t->shape[2] + nc) * L;
        if (rotary_mode == 0) {
          half_mode_row(x, cos_t, sin_t, xrow + start, crow, L, x64, backward);
          continue;
        }
        for (int64_t i = 0; i < L / 2; ++i) {
          int64_t j0 = xrow + start + 2 * i, j1 = j0 + 1; /* pair counted from the slice start */
          float a = load_f32(x, j0);
          float bb = load_f32(x, j1);
          float c0 = load_f32(cos_t, crow + 2 * i), c1 = load_f32(cos_t, crow + 2 * i + 1);
          float s0 = load_f32(sin_t, crow + 2 * i), s1 = load_f32(sin_t, crow + 2 * i + 1);
          float y0, y1;
          if (!backward) {
            /* y = x*cos + x_rotate*sin with x_rotate = (-b, a) on the pair */
            float p0 = a * c0;
            float q0 = (-bb) * s0;
            y0 = p0 + q0;
            float p1 = bb * c1;
            float q1 = a * s1;
            y1 = p1 + q1;
            if (x64) {
              x64[j0] = (double)a * (double)c0 + (-(double)bb) * (double)s0;
              x64[j1] = (double)bb * (double)c1 + (double)a * (double)s1;
            }
          } else {
            /* gradient: the pair map is y = M x with M = [[c0, -s0], [s1, c1]], so
             * dx = M^T g = (c0*g0 + s1*g1, c1*g1 - s0*g0); here (a, bb) = (g0, g1) */
            float p0 = a * c0;
            float q0 = bb * s1;
            y0 = p0 + q0;
            float p1 = bb * c1;
            float q1 = a * s0;
            y1 = p1 - q1;
            if (x64) {
              x64[j0] = (double)a * (double)c0 + (double)bb * (double)s1;
              x64[j1] = (double)bb * (double)c1 - (double)a * (double)s0;
            }
          }
          store_rounded(x, j0, y0);
          store_rounded(x, j1, y1);
        }
      }
  return ORO_OK;
}

int oro_rope_partial_inplace(const oro_tensor *x, const oro_tensor *cos_t, const oro_tensor *sin_t,
                             int64_t rotary_mode, const int64_t *partial_slice,
                             int64_t partial_slice_len, double *x64) {
  return partial_inplace(x, cos_t, sin_t, rotary_mode, partial_slice, partial_slice_len, x64, 0);
}

/* Backward of operation A, in place on the incoming gradient g (same shapes, validation and
 * no-op rules as the forward).  [IPRM §Python 接口与自动微分]: the training path computes the
 * gradient of x with a backward op, cos/sin get no gradient, and empty tensors and empty
 * slices are no-ops.  The pages give no formula; the gradient of the linear pair map above
 * is its transpose.  Elements outside the slice pass the gradient through unchanged. */
int oro_rope_partial_inplace_backward(const oro_tensor *g, const oro_tensor *cos_t,
                                      const oro_tensor *sin_t, int64_t rotary_mode,
                                      const int64_t *partial_slice, int64_t partial_slice_len,
                                      double *g64) {
  return partial_inplace(g, cos_t, sin_t, rotary_mode, partial_slice, partial_slice_len, g64, 1);
}

/* ==========================================================================================
 * Operation B: RoPE with a cos/sin cache (rope and mrope modes, GPT-NeoX or GPT-J style).
 *   [RSCC §设计动机]            gather cosSin = cosSinCache[positions], split into cos | sin,
 *                               rotate the first rotaryDim of each head, pass the rest through;
 *   [RSCC §rope 模式：标准位置编码]  positions [numTokens]; mropeSection null -> rope;
 *   [RSCC §mrope 模式：多模态位置编码] positions [m, numTokens]; cos/sin stitched by sections;
 *   [RSCC §rotate_half（GPT-NeoX style）旋转模式]   pairs (i, i + rotaryDim/2);
 *   [RSCC §rotate_interleaved（GPT-J style）旋转模式] pairs (2i, 2i+1) (reading R8);
 *   [RSCC §约束说明]            2-D q/k/cache, equal dtypes, 64-byte aligned headSize and
 *                               rotaryDim, rotaryDim <= headSize, 2*sum(mropeSection) == rotaryDim,
 *                               positions < maxSeqLen;
 *   [RSCC §入参校验逻辑]        null / dtype / shape / mropeSection checks and the whitelist.
 * Error codes follow [IPRM §返回值与错误码] (this page's own table did not survive).
 * ========================================================================================== */

static const int64_t kMropeWhitelist[5][4] = {
    {16, 24, 24, 0}, {8, 12, 12, 0}, {24, 20, 20, 0}, {11, 11, 10, 0}, {16, 16, 16, 16}};
static const int kMropeWhitelistLen[5] = {3, 3, 3, 3, 4};

/* byte range [lo, hi) touched by a 2-D tensor with non-negative strides */
static void byte_range(const oro_tensor *t, uintptr_t *lo, uintptr_t *hi) {
  int es = elem_size(t->dtype);
  int64_t last = 0;
  for (int d = 0; d < t->ndim; ++d) last += (t->shape[d] - 1) * t->stride[d];
  *lo = (uintptr_t)t->data;
  *hi = (uintptr_t)t->data + (uintptr_t)((last + 1) * es);
}

static int ranges_overlap(const oro_tensor *a, const oro_tensor *b) {
  uintptr_t alo, ahi, blo, bhi;
  byte_range(a, &alo, &ahi);
  byte_range(b, &blo, &bhi);
  return alo < bhi && blo < ahi;
}

static int same_layout(const oro_tensor *a, const oro_tensor *b) {
  if (a->data != b->data || a->ndim != b->ndim) return 0;
  for (int d = 0; d < a->ndim; ++d)
    if (a->shape[d] != b->shape[d] || (a->shape[d] > 1 && a->stride[d] != b->stride[d])) return 0;
  return 1;
}

static int cos_sin_cache(const oro_tensor *positions, const oro_tensor *query_in,
                         const oro_tensor *key_in, const oro_tensor *cache,
                         const int64_t *mrope_section, int64_t mrope_section_len,
                         int64_t head_size, int is_neox_style, int64_t cache_mode,
                         const oro_tensor *query_out, const oro_tensor *key_out, double *q64,
                         double *k64) {
  const oro_tensor *all[6] = {positions, query_in, key_in, cache, query_out, key_out};
  for (int i = 0; i < 6; ++i)
    if (!all[i]) return fail(ORO_ERR_PARAM_NULLPTR, "a tensor argument is null");
  if (!mrope_section && mrope_section_len > 0)
    return fail(ORO_ERR_PARAM_NULLPTR, "mropeSection is null but its length is not 0");
  if (mrope_section_len < 0) return fail(ORO_ERR_PARAM_INVALID, "negative mropeSection length");
  for (int i = 0; i < 6; ++i)
    if (shape_ok(all[i]) && numel(all[i]) > 0 && !all[i]->data)
      return fail(ORO_ERR_PARAM_NULLPTR, "a non-empty tensor has a null data pointer");

  /* dtypes */
  if (positions->dtype != ORO_I64) return fail(ORO_ERR_PARAM_INVALID, "positions must be int64");
  if (!is_float_dtype(query_in->dtype)) return fail(ORO_ERR_PARAM_INVALID, "queryIn dtype unsupported");
  if (key_in->dtype != query_in->dtype || cache->dtype != query_in->dtype ||
      query_out->dtype != query_in->dtype || key_out->dtype != query_in->dtype)
    return fail(ORO_ERR_PARAM_INVALID, "dtypes of keyIn/cosSinCache/outputs must equal queryIn's");

  /* shapes */
  const oro_tensor *two_d[5] = {query_in, key_in, cache, query_out, key_out};
  for (int i = 0; i < 5; ++i)
    if (!shape_ok(two_d[i]) || two_d[i]->ndim != 2)
      return fail(ORO_ERR_PARAM_INVALID, "queryIn, keyIn, cosSinCache and outputs must be 2-D");
  for (int i = 0; i < 6; ++i)
    if (shape_ok(all[i]) && beyond_limits(all[i]))
      return fail(ORO_ERR_PARAM_INVALID, "tensor too large to exist");
  for (int i = 0; i < 3; ++i)
    if (two_d[i]->shape[0] <= 0 || two_d[i]->shape[1] <= 0)
      return fail(ORO_ERR_PARAM_INVALID, "queryIn, keyIn and cosSinCache must be non-empty");
  if (key_in->shape[0] != query_in->shape[0])
    return fail(ORO_ERR_PARAM_INVALID, "keyIn and queryIn token counts differ");
  for (int d = 0; d < 2; ++d)
    if (query_out->shape[d] != query_in->shape[d] || key_out->shape[d] != key_in->shape[d])
      return fail(ORO_ERR_PARAM_INVALID, "output shapes must equal input shapes");
  const int64_t T = query_in->shape[0];
  const int64_t rd = cache->shape[1];
  const int64_t max_seq = cache->shape[0];

  /* mropeSection (reading R9) */
  int mrope = 0;
  int64_t nsec = 0;
  int64_t sec[4] = {0, 0, 0, 0};
  if (mrope_section_len > 0) {
    if (mrope_section_len != 3 && mrope_section_len != 4)
      return fail(ORO_ERR_PARAM_INVALID, "mropeSection must have 3 or 4 elements");
    int64_t sum = 0;
    for (int64_t i = 0; i < mrope_section_len; ++i) {
      if (mrope_section[i] < 0 || mrope_section[i] > rd)
        return fail(ORO_ERR_PARAM_INVALID, "mropeSection element outside [0, rotaryDim]");
      sum += mrope_section[i];
    }
    if (mrope_section[0] > 0) {
      if (2 * sum != rd) return fail(ORO_ERR_PARAM_INVALID, "2*sum(mropeSection) != rotaryDim");
      int listed = 0;
      for (int w = 0; w < 5 && !listed; ++w) {
        if (kMropeWhitelistLen[w] != mrope_section_len) continue;
        int eq = 1;
        for (int64_t i = 0; i < mrope_section_len; ++i) eq &= (kMropeWhitelist[w][i] == mrope_section[i]);
        listed = eq;
      }
      if (!listed) return fail(ORO_ERR_PARAM_INVALID, "mropeSection is not a supported list");
      mrope = 1;
      nsec = mrope_section_len;
      for (int64_t i = 0; i < nsec; ++i) sec[i] = mrope_section[i];
    }
  }

  /* cacheMode ([RSCC §V2 接口：cacheMode 扩展]): 0 sectioned, 1 interleaved; the 4-section list
   * allows 0 only.  In rope mode the value has no effect. */
  if (cache_mode != 0 && cache_mode != 1)
    return fail(ORO_ERR_PARAM_INVALID, "cacheMode must be 0 or 1");
  if (mrope && cache_mode == 1 && nsec == 4)
    return fail(ORO_ERR_PARAM_INVALID, "cacheMode 1 needs a 3-section mropeSection");

  /* headSize and rotaryDim: 64-byte multiples, rotaryDim <= headSize */
  const int es = elem_size(query_in->dtype);
  const int64_t align = 64 / es;
  if (head_size <= 0 || head_size % align != 0)
    return fail(ORO_ERR_PARAM_INVALID, "headSize must be a positive multiple of 64 bytes");
  if (query_in->shape[1] % head_size != 0 || key_in->shape[1] % head_size != 0)
    return fail(ORO_ERR_PARAM_INVALID, "queryIn/keyIn widths are not multiples of headSize");
  if (rd > head_size || rd % align != 0)
    return fail(ORO_ERR_PARAM_INVALID, "rotaryDim must be a 64-byte multiple no larger than headSize");

  /* positions */
  if (!shape_ok(positions)) return fail(ORO_ERR_PARAM_INVALID, "positions shape invalid");
  if (!mrope) {
    if (positions->ndim != 1 || positions->shape[0] != T)
      return fail(ORO_ERR_PARAM_INVALID, "rope mode needs positions of shape [numTokens]");
  } else {
    if (positions->ndim != 2 || positions->shape[0] != nsec || positions->shape[1] != T)
      return fail(ORO_ERR_PARAM_INVALID, "mrope mode needs positions of shape [m, numTokens]");
  }

  /* strides: unit inner strides on q/k/cache, non-negative row strides, contiguous outputs */
  for (int i = 0; i < 3; ++i)
    if (two_d[i]->stride[1] != 1 || two_d[i]->stride[0] < 0)
      return fail(ORO_ERR_PARAM_INVALID, "inputs need unit inner stride and non-negative row stride");
  for (int d = 0; d < positions->ndim; ++d)
    if (positions->stride[d] < 0) return fail(ORO_ERR_PARAM_INVALID, "negative positions stride");
  if (!contiguous(query_out) || !contiguous(key_out))
    return fail(ORO_ERR_PARAM_INVALID, "queryOut/keyOut must be contiguous");

  /* outputs may alias their own input exactly, nothing else may overlap an output */
  if (ranges_overlap(query_out, key_out)) return fail(ORO_ERR_PARAM_INVALID, "queryOut and keyOut overlap");
  const oro_tensor *ins[4] = {positions, query_in, key_in, cache};
  const oro_tensor *outs[2] = {query_out, key_out};
  for (int o = 0; o < 2; ++o)
    for (int i = 0; i < 4; ++i) {
      if (!ranges_overlap(outs[o], ins[i])) continue;
      if ((o == 0 && i == 1 && same_layout(query_out, query_in)) ||
          (o == 1 && i == 2 && same_layout(key_out, key_in)))
        continue;
      return fail(ORO_ERR_PARAM_INVALID, "an output overlaps an input");
    }

  /* positions inside the cache (reading R11): checked before anything is written */
  for (int64_t k = 0; k < (mrope ? nsec : 1); ++k)
    for (int64_t t = 0; t < T; ++t) {
      int64_t p = mrope ? load_i64(positions, k * positions->stride[0] + t * positions->stride[1])
                        : load_i64(positions, t * positions->stride[0]);
      if (p < 0 || p >= max_seq) return fail(ORO_ERR_OUTSIDE_CONTRACT, "position outside the cache");
    }

  const int64_t half = rd / 2;
  const int64_t nq = query_in->shape[1] / head_size, nk = key_in->shape[1] / head_size;
  /* one token's gathered cos and sin (rotaryDim/2 each) and one head's rotated inputs
   * (rotaryDim): the pages bound rotaryDim only by headSize, so these are sized per call */
  float *cs_cos = malloc((size_t)rd * sizeof(float));
  float *vin = malloc((size_t)rd * sizeof(float));
  if (!cs_cos || !vin) {
    free(cs_cos);
    free(vin);
    return fail(ORO_ERR_OUT_OF_MEMORY, "oracle: no host memory for one row of rotaryDim");
  }
  float *cs_sin = cs_cos + half;

  for (int64_t t = 0; t < T; ++t) {
    /* gather the cache row(s) and split into cos | sin; mrope stitches the
     * sections: element i of cos/sin comes from the position row whose section holds i */
    for (int64_t i = 0; i < half; ++i) {
      int64_t row_sel = 0;
      if (mrope && cache_mode == 0) {
        /* sectioned: element i takes the row of the section that holds it */
        int64_t acc = 0;
        for (int64_t k = 0; k < nsec; ++k) {
          acc += sec[k];
          if (i < acc) { row_sel = k; break; }
        }
      } else if (mrope) {
        /* interleaved ([RSCC §V2 接口：cacheMode 扩展]): start from row 0, then the elements
         * 1, 4, 7, ... below 3*mropeSection[1] come from row 1 and 2, 5, 8, ... below the same
         * bound from row 2 (the bound printed for both; for every accepted list it selects the
         * same elements as 3*mropeSection[2] would, the slices ending at rotaryDim/2) */
        if (i % 3 == 1 && i < 3 * sec[1]) row_sel = 1;
        else if (i % 3 == 2 && i < 3 * sec[1]) row_sel = 2;
      }
      int64_t p = mrope ? load_i64(positions, row_sel * positions->stride[0] + t * positions->stride[1])
                        : load_i64(positions, t * positions->stride[0]);
      cs_cos[i] = load_f32(cache, p * cache->stride[0] + i);
      cs_sin[i] = load_f32(cache, p * cache->stride[0] + half + i);
    }
    /* rotate: every query head, then every key head */
    for (int which = 0; which < 2; ++which) {
      const oro_tensor *in = which == 0 ? query_in : key_in;
      const oro_tensor *out = which == 0 ? query_out : key_out;
      double *o64 = which == 0 ? q64 : k64;
      int64_t nh = which == 0 ? nq : nk;
      for (int64_t h = 0; h < nh; ++h) {
        int64_t ib = t * in->stride[0] + h * head_size;      /* input head base   */
        int64_t ob = t * (nh * head_size) + h * head_size;   /* output head base  */
        /* the rotated part: read every input of the head first, since an exactly aliased
         * output may overwrite it */
        for (int64_t j = 0; j < rd; ++j) vin[j] = load_f32(in, ib + j);
        for (int64_t i = 0; i < half; ++i) {
          int64_t ja, jb;
          if (is_neox_style) { ja = i; jb = i + half; }       /* x1 = first half, x2 = second */
          else { ja = 2 * i; jb = 2 * i + 1; }                /* x1 = even, x2 = odd          */
          float a = vin[ja], bb = vin[jb], c = cs_cos[i], s = cs_sin[i];
          float o1 = a * c - bb * s;   /* o1 = x1*cos - x2*sin: two products, one difference */
          float o2 = bb * c + a * s;   /* o2 = x2*cos + x1*sin                               */
          if (o64) {
            o64[ob + ja] = (double)a * (double)c - (double)bb * (double)s;
            o64[ob + jb] = (double)bb * (double)c + (double)a * (double)s;
          }
          store_rounded(out, ob + ja, o1);
          store_rounded(out, ob + jb, o2);
        }
        /* the pass-through part, bit for bit */
        for (int64_t j = rd; j < head_size; ++j) {
          if (o64) o64[ob + j] = (double)load_f32(in, ib + j);
          copy_bits(out, ob + j, in, ib + j);
        }
      }
    }
  }
  free(cs_cos);
  free(vin);
  return ORO_OK;
}

int oro_rope_with_cos_sin_cache(const oro_tensor *positions, const oro_tensor *query_in,
                                const oro_tensor *key_in, const oro_tensor *cache,
                                const int64_t *mrope_section, int64_t mrope_section_len,
                                int64_t head_size, int is_neox_style,
                                const oro_tensor *query_out, const oro_tensor *key_out,
                                double *q64, double *k64) {
  return cos_sin_cache(positions, query_in, key_in, cache, mrope_section, mrope_section_len,
                       head_size, is_neox_style, 0, query_out, key_out, q64, k64);
}

/* The V2 form with the cacheMode argument ([RSCC §V2 接口：cacheMode 扩展]); cacheMode 0 is the
 * call above. */
int oro_rope_with_cos_sin_cache_v2(const oro_tensor *positions, const oro_tensor *query_in,
                                   const oro_tensor *key_in, const oro_tensor *cache,
                                   const int64_t *mrope_section, int64_t mrope_section_len,
                                   int64_t head_size, int is_neox_style, int64_t cache_mode,
                                   const oro_tensor *query_out, const oro_tensor *key_out,
                                   double *q64, double *k64) {
  return cos_sin_cache(positions, query_in, key_in, cache, mrope_section, mrope_section_len,
                       head_size, is_neox_style, cache_mode, query_out, key_out, q64, k64);
}
