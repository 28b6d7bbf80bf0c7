// rope_kernels.hip -- gfx950 (MI355X) kernels and C-ABI entry points of librope_amd.so.
//
// Both operations are elementwise rotations of (pairs of) activations by cos/sin values: a
// few flops per 4+ bytes moved, so they are bound by HBM bandwidth.  There is no contraction
// here (no MFMA); the kernels are built around wide, coalesced 16-byte accesses, the pairs of
// a rotation held in one lane's registers (or, in half mode, in two lanes of one wavefront),
// float32 arithmetic with one rounding per product and per sum, and one rounding to the
// storage type.
//
// Pages:
//   [IPRM] "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码
//           接口详解与实现剖析"
//   [RSCC] "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的
//           计算原理与 aclnn 两段式调用实战"
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "rope.h"
#include "rope_plan.h"

// Products and sums are separate float32 operations, never fused into one multiply-add: the
// formulas of both pages are two products and one sum, each rounded.
#pragma clang fp contract(off)

namespace ropeamd {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---- storage types <-> float32 ------------------------------------------------------------
// Decoding is exact; encoding rounds to nearest even (gfx950's v_cvt_pk_bf16_f32 and
// v_cvt_f16_f32 under the default round-to-nearest-even mode).

template <typename T>
struct Io;

template <>
struct Io<float> {
  static constexpr int kPer16 = 4;
  static constexpr int kPerWord = 1;
  using raw = uint32_t;
  __device__ static void word_to_floats(uint32_t w, float *f) { f[0] = __uint_as_float(w); }
  __device__ static uint32_t floats_to_word(const float *f) { return __float_as_uint(f[0]); }
  __device__ static void unpack(const uint4 &v, float *f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static uint4 pack(const float *f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
  __device__ static float from_raw(raw r) { return __uint_as_float(r); }
  __device__ static float load1(const void *p, int64_t i) {
    return static_cast<const float *>(p)[i];
  }
  __device__ static void store1(void *p, int64_t i, float v) { static_cast<float *>(p)[i] = v; }
};

template <>
struct Io<__bf16> {
  static constexpr int kPer16 = 8;
  static constexpr int kPerWord = 2;
  using raw = uint16_t;
  __device__ static void word_to_floats(uint32_t w, float *f) { unpack_word(w, f); }
  __device__ static uint32_t floats_to_word(const float *f) { return pack_word(f[0], f[1]); }
  __device__ static void unpack_word(uint32_t w, float *f) {
    f[0] = __uint_as_float(w << 16);
    f[1] = __uint_as_float(w & 0xffff0000u);
  }
  __device__ static uint32_t pack_word(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  __device__ static void unpack(const uint4 &v, float *f) {
    unpack_word(v.x, f);
    unpack_word(v.y, f + 2);
    unpack_word(v.z, f + 4);
    unpack_word(v.w, f + 6);
  }
  __device__ static uint4 pack(const float *f) {
    return make_uint4(pack_word(f[0], f[1]), pack_word(f[2], f[3]), pack_word(f[4], f[5]),
                      pack_word(f[6], f[7]));
  }
  __device__ static float from_raw(raw r) { return __uint_as_float(uint32_t(r) << 16); }
  __device__ static float load1(const void *p, int64_t i) {
    return from_raw(static_cast<const uint16_t *>(p)[i]);
  }
  __device__ static void store1(void *p, int64_t i, float v) {
    static_cast<uint16_t *>(p)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  }
};

template <>
struct Io<_Float16> {
  static constexpr int kPer16 = 8;
  static constexpr int kPerWord = 2;
  using raw = uint16_t;
  __device__ static void word_to_floats(uint32_t w, float *f) { unpack_word(w, f); }
  __device__ static uint32_t floats_to_word(const float *f) { return pack_word(f[0], f[1]); }
  __device__ static void unpack_word(uint32_t w, float *f) {
    f16x2 h = __builtin_bit_cast(f16x2, w);
    f[0] = static_cast<float>(h.x);
    f[1] = static_cast<float>(h.y);
  }
  __device__ static uint32_t pack_word(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  __device__ static void unpack(const uint4 &v, float *f) {
    unpack_word(v.x, f);
    unpack_word(v.y, f + 2);
    unpack_word(v.z, f + 4);
    unpack_word(v.w, f + 6);
  }
  __device__ static uint4 pack(const float *f) {
    return make_uint4(pack_word(f[0], f[1]), pack_word(f[2], f[3]), pack_word(f[4], f[5]),
                      pack_word(f[6], f[7]));
  }
  __device__ static float from_raw(raw r) {
    return static_cast<float>(__builtin_bit_cast(_Float16, r));
  }
  __device__ static float load1(const void *p, int64_t i) {
    return static_cast<float>(static_cast<const _Float16 *>(p)[i]);
  }
  __device__ static void store1(void *p, int64_t i, float v) {
    static_cast<_Float16 *>(p)[i] = static_cast<_Float16>(v);
  }
};

// 16-byte raw vector (a native vector type, accepted by the non-temporal builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load/store; NT marks the access non-temporal (streamed data that is touched once:
// it is not kept in the caches, which leaves them to data that is reused).
template <bool NT>
__device__ inline u32x4 ld16(const void *p) {
  const u32x4 *q = static_cast<const u32x4 *>(p);
  if constexpr (NT) return __builtin_nontemporal_load(q);
  return *q;
}

template <bool NT>
__device__ inline void st16(void *p, u32x4 v) {
  u32x4 *q = static_cast<u32x4 *>(p);
  if constexpr (NT) __builtin_nontemporal_store(v, q);
  else *q = v;
}

__device__ inline uint4 to_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ inline u32x2 ld8(const void *p) {
  const u32x2 *q = static_cast<const u32x2 *>(p);
  if constexpr (NT) return __builtin_nontemporal_load(q);
  return *q;
}

template <bool NT>
__device__ inline void st8(void *p, u32x2 v) {
  u32x2 *q = static_cast<u32x2 *>(p);
  if constexpr (NT) __builtin_nontemporal_store(v, q);
  else *q = v;
}

// N consecutive elements starting at element `i` of `p`, as float32.  VEC: the address is
// aligned to the access size and N * sizeof(T) is 8 bytes or a multiple of 16, so whole
// 8- or 16-byte loads are used; otherwise one element at a time.
template <typename T, int N, bool VEC, bool NT>
__device__ inline void load_n(const void *p, int64_t i, float *f) {
  constexpr int kBytes = N * int(sizeof(T));
  constexpr int kPW = Io<T>::kPerWord;
  if constexpr (VEC && kBytes % 16 == 0) {
    const char *q = reinterpret_cast<const char *>(static_cast<const T *>(p) + i);
#pragma unroll
    for (int c = 0; c < kBytes / 16; ++c) {
      const u32x4 v = ld16<NT>(q + 16 * c);
      Io<T>::word_to_floats(v.x, f + (4 * c + 0) * kPW);
      Io<T>::word_to_floats(v.y, f + (4 * c + 1) * kPW);
      Io<T>::word_to_floats(v.z, f + (4 * c + 2) * kPW);
      Io<T>::word_to_floats(v.w, f + (4 * c + 3) * kPW);
    }
  } else if constexpr (VEC && kBytes == 8) {
    const u32x2 v = ld8<NT>(static_cast<const T *>(p) + i);
    Io<T>::word_to_floats(v.x, f);
    Io<T>::word_to_floats(v.y, f + kPW);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) f[e] = Io<T>::load1(p, i + e);
  }
}

template <typename T, int N, bool VEC, bool NT>
__device__ inline void store_n(void *p, int64_t i, const float *f) {
  constexpr int kBytes = N * int(sizeof(T));
  constexpr int kPW = Io<T>::kPerWord;
  if constexpr (VEC && kBytes % 16 == 0) {
    char *q = reinterpret_cast<char *>(static_cast<T *>(p) + i);
#pragma unroll
    for (int c = 0; c < kBytes / 16; ++c)
      st16<NT>(q + 16 * c, u32x4{Io<T>::floats_to_word(f + (4 * c + 0) * kPW),
                                 Io<T>::floats_to_word(f + (4 * c + 1) * kPW),
                                 Io<T>::floats_to_word(f + (4 * c + 2) * kPW),
                                 Io<T>::floats_to_word(f + (4 * c + 3) * kPW)});
  } else if constexpr (VEC && kBytes == 8) {
    st8<NT>(static_cast<T *>(p) + i,
            u32x2{Io<T>::floats_to_word(f), Io<T>::floats_to_word(f + kPW)});
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) Io<T>::store1(p, i + e, f[e]);
  }
}

// BYTES (8 or a multiple of 16) raw bytes in 32-bit words: lets a lane issue all of its
// loads before converting any of them (converting at once makes the compiler wait for each
// load in turn to keep fewer registers live).
template <int BYTES>
struct Words {
  static_assert(BYTES == 8 || BYTES % 16 == 0, "8 bytes or a multiple of 16");
  uint32_t w[BYTES / 4];
};

template <int BYTES, bool NT>
__device__ inline void load_words(const void *p, Words<BYTES> &r) {
  if constexpr (BYTES == 8) {
    const u32x2 v = ld8<NT>(p);
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else {
#pragma unroll
    for (int c = 0; c < BYTES / 16; ++c) {
      const u32x4 v = ld16<NT>(static_cast<const char *>(p) + 16 * c);
      r.w[4 * c] = v.x;
      r.w[4 * c + 1] = v.y;
      r.w[4 * c + 2] = v.z;
      r.w[4 * c + 3] = v.w;
    }
  }
}

template <typename T, int N>
__device__ inline void words_to_floats(const Words<N * int(sizeof(T))> &r, float *f) {
#pragma unroll
  for (int q = 0; q < N * int(sizeof(T)) / 4; ++q)
    Io<T>::word_to_floats(r.w[q], f + q * Io<T>::kPerWord);
}

// Raw copy of N elements (pass-through data is moved as bits, never converted).
template <typename T, int N, bool VEC>
struct RawN {
  u32x4 v[VEC ? (N * int(sizeof(T)) + 15) / 16 : 1];
  typename Io<T>::raw e[VEC ? 1 : N];
};

template <typename T, int N, bool VEC, bool NT>
__device__ inline void load_raw(const void *p, int64_t i, RawN<T, N, VEC> &r) {
  if constexpr (VEC) {
    const char *q = reinterpret_cast<const char *>(static_cast<const T *>(p) + i);
#pragma unroll
    for (int c = 0; c < (N * int(sizeof(T))) / 16; ++c) r.v[c] = ld16<NT>(q + 16 * c);
  } else {
    const typename Io<T>::raw *q = static_cast<const typename Io<T>::raw *>(p) + i;
#pragma unroll
    for (int e = 0; e < N; ++e) r.e[e] = q[e];
  }
}

template <typename T, int N, bool VEC, bool NT>
__device__ inline void store_raw(void *p, int64_t i, const RawN<T, N, VEC> &r) {
  if constexpr (VEC) {
    char *q = reinterpret_cast<char *>(static_cast<T *>(p) + i);
#pragma unroll
    for (int c = 0; c < (N * int(sizeof(T))) / 16; ++c) st16<NT>(q + 16 * c, r.v[c]);
  } else {
    typename Io<T>::raw *q = static_cast<typename Io<T>::raw *>(p) + i;
#pragma unroll
    for (int e = 0; e < N; ++e) q[e] = r.e[e];
  }
}

template <typename T, int N, bool VEC>
__device__ inline void raw_to_float(const RawN<T, N, VEC> &r, float *f) {
  if constexpr (VEC) {
#pragma unroll
    for (int c = 0; c < (N * int(sizeof(T))) / 16; ++c)
      Io<T>::unpack(to_uint4(r.v[c]), f + c * Io<T>::kPer16);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) f[e] = Io<T>::from_raw(r.e[e]);
  }
}

// Word q (kPerWord elements) of a raw vector, as float32; and its inverse (one rounding).
template <typename T, int N, bool VEC>
__device__ inline void raw_word_to_float(const RawN<T, N, VEC> &r, int q, float *f) {
  if constexpr (VEC) {
    const u32x4 v = r.v[q / 4];
    const int j = q % 4;
    Io<T>::word_to_floats(j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w, f);
  } else {
#pragma unroll
    for (int e = 0; e < Io<T>::kPerWord; ++e) f[e] = Io<T>::from_raw(r.e[q * Io<T>::kPerWord + e]);
  }
}

template <typename T, int N, bool VEC>
__device__ inline void float_to_raw_word(const float *f, int q, RawN<T, N, VEC> &r) {
  if constexpr (VEC) {
    const uint32_t w = Io<T>::floats_to_word(f);
    const int j = q % 4;
    if (j == 0) r.v[q / 4].x = w;
    else if (j == 1) r.v[q / 4].y = w;
    else if (j == 2) r.v[q / 4].z = w;
    else r.v[q / 4].w = w;
  } else {
#pragma unroll
    for (int e = 0; e < Io<T>::kPerWord; ++e) {
      float one = f[e];
      Io<T>::store1(&r.e[q * Io<T>::kPerWord + e], 0, one);
    }
  }
}

__device__ inline uint32_t fdiv(const FastDiv &f, uint32_t n) {
  const uint32_t t = __umulhi(f.m, n);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

// One pair (x0, x1) of [IPRM §计算原理与公式]: (x[2i], x[2i+1]) in interleave mode (reading:
// x_rotate = (-x[2i+1], x[2i]) per pair), (x[i], x[i + L/2]) in half mode; c0, s0 are the
// cos/sin entries of x0's position and c1, s1 those of x1's:
//   forward  y0 = x0*c0 + (-x1)*s0,  y1 = x1*c1 + x0*s1;
//   backward (transpose of the pair map, [IPRM §Python 接口与自动微分]):
//            g0' = g0*c0 + g1*s1,    g1' = g1*c1 - g0*s0.
template <bool BWD>
__device__ inline void rotate_pair(float a, float b, float c0, float c1, float s0, float s1,
                                   float &y0, float &y1) {
  if constexpr (!BWD) {
    y0 = a * c0 - b * s0;
    y1 = b * c1 + a * s1;
  } else {
    y0 = a * c0 + b * s1;
    y1 = b * c1 - a * s0;
  }
}

// ============================================================================================
// K1: in-place partial RoPE ([IPRM §计算原理与公式], [IPRM §partial_slice 局部旋转机制]).
// Interleave mode: a lane owns a chunk of V slice elements (V/2 pairs); chunks of one row are
// adjacent lanes, so a wavefront reads and writes whole 16-byte-aligned runs of each row's
// slice.  HALF (rotary_mode 0, [IPRM §参数说明]; x1, x2 the two halves of the slice,
// x_rotate = cat(-x2, x1)): a lane owns chunk u of the first half and chunk u of the second,
// so every pair (i, i + L/2) is lane-local and both halves are read as contiguous runs.
// XCH (half mode, 1..16 chunks per half): a lane owns one chunk of one half and reads its
// pair partners from lane (lane ^ xch) with ds_bpermute, xch being the chunk count of a half
// rounded up to a power of two (PAD when that rounds up: the extra lanes carry no chunk), so
// the launch has about as many lanes, and each lane as few loads, as in interleave mode.
// NHL = 2 or 4 (cos/sin broadcast over the heads): the lane owns its chunk in NHL consecutive
// heads of one (b, s) and loads the cos/sin chunk once for all of them.  Elements outside
// [start, end) are never touched.  cos/sin rows are addressed with zero strides on broadcast
// dims (BSND, BS1D, B1ND, B11D, 111D and mixed forms).  BWD runs the transpose of the pair map
// on an incoming gradient (same access pattern).  x is streamed (non-temporal); cos/sin are
// streamed too when each of their rows is read by one lane group, else (broadcast) loaded
// normally so that the caches serve the repeats.
// ============================================================================================
// One lane item: chunk `chunk` of the NHL x rows starting at row r * NHL, whose cos/sin row
// is that of (b, s, head g * NHL).
template <typename XT, typename CT, bool VEC, int NHL, bool CNT, bool BWD, bool HALF, bool XCH,
          bool PAD>
// xrow: first element of the item's row group in x (r * nhl * D); crow_el: first element of
// its cos/sin row (crow * L).
__device__ __forceinline__ void inplace_item(const InplacePlan &p, uint64_t chunk, int64_t xrow,
                                             int64_t crow_el) {
  // one 16-byte access per lane for the wider of x and cos/sin, 8 bytes for the narrower;
  // element access: one pair (2 elements) in interleave mode, one element per half in HALF
  constexpr int V =
      VEC ? 16 / (sizeof(XT) > sizeof(CT) ? int(sizeof(XT)) : int(sizeof(CT))) : (HALF ? 1 : 2);
  constexpr int NH = HALF && !XCH ? 2 : 1;  // chunks per head: one, or one in each half
  const int64_t hoff = HALF ? p.L / 2 : 0;  // offset of the second half
  // element offset of the chunk in the slice.  PAD (XCH with a half's chunk count below the
  // power of two xch): chunk c of the first half or of the second (chunk >= xch), the lanes
  // past a half's last chunk loading that chunk and storing nothing
  int64_t elem = int64_t(chunk) * V;
  bool owns = true;
  if constexpr (XCH && PAD) {
    const uint32_t c = uint32_t(chunk) & (p.xch - 1);
    owns = c < p.xch_cph;
    elem = (chunk >= p.xch ? p.L / 2 : 0) + int64_t(owns ? c : p.xch_cph - 1) * V;
  }
  const int64_t coff = crow_el + elem;
  const int64_t x0 = xrow + p.start + elem;
  float xv[NHL][NH][V], cv[NH][V], sv[NH][V];
  float xpv[XCH ? NHL : 1][V], spv[XCH && BWD ? V : 1];  // XCH: the partner lane's x, sin
  if constexpr (VEC) {
    constexpr int XB = V * int(sizeof(XT)), CB = V * int(sizeof(CT));
    Words<XB> xr[NHL][NH];
    Words<CB> cr[NH], sr[NH];
#pragma unroll
    for (int j = 0; j < NHL; ++j)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        load_words<XB, true>(static_cast<const XT *>(p.x) + x0 + j * p.D + hh * hoff, xr[j][hh]);
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      load_words<CB, CNT>(static_cast<const CT *>(p.cos) + coff + hh * hoff, cr[hh]);
      load_words<CB, CNT>(static_cast<const CT *>(p.sin) + coff + hh * hoff, sr[hh]);
    }
    if constexpr (XCH) {
      // The pair partners of this lane's chunk sit in the same chunk of the other half,
      // owned by lane (lane ^ xch) of this wavefront (a row's 2 * xch lanes are consecutive
      // and aligned).  The raw words are exchanged: forward needs the partner's x, the
      // gradient also the partner's sin.
      const int src = int((__lane_id() ^ p.xch) << 2);
#pragma unroll
      for (int j = 0; j < NHL; ++j) {
        Words<XB> xw;
#pragma unroll
        for (int q = 0; q < XB / 4; ++q)
          xw.w[q] = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(xr[j][0].w[q])));
        words_to_floats<XT, V>(xw, xpv[j]);
      }
      if constexpr (BWD) {
        Words<CB> sw;
#pragma unroll
        for (int q = 0; q < CB / 4; ++q)
          sw.w[q] = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(sr[0].w[q])));
        words_to_floats<CT, V>(sw, spv);
      }
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
      for (int j = 0; j < NHL; ++j) words_to_floats<XT, V>(xr[j][hh], xv[j][hh]);
      words_to_floats<CT, V>(cr[hh], cv[hh]);
      words_to_floats<CT, V>(sr[hh], sv[hh]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NHL; ++j)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        load_n<XT, V, false, true>(p.x, x0 + j * p.D + hh * hoff, xv[j][hh]);
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      load_n<CT, V, false, CNT>(p.cos, coff + hh * hoff, cv[hh]);
      load_n<CT, V, false, CNT>(p.sin, coff + hh * hoff, sv[hh]);
    }
  }
  if constexpr (XCH) {
    static_assert(HALF && VEC, "the lane exchange is a half-mode vector path");
    const bool second = chunk >= p.xch;  // this chunk lies in the second half
#pragma unroll
    for (int j = 0; j < NHL; ++j) {
      // first half: forward x*c - x'*s, gradient x*c + x'*s'; second half: the other signs
      // (x' and s' the partner's values; the same products and sums as the pair map)
      float y[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float pr = xv[j][0][e] * cv[0][e];
        const float qr = xpv[j][e] * (BWD ? spv[e] : sv[0][e]);
        y[e] = (second == BWD) ? pr - qr : pr + qr;
      }
      if (owns) store_n<XT, V, VEC, true>(p.x, x0 + j * p.D, y);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < NHL; ++j) {
    if constexpr (HALF) {
      float ya[V], yb[V];
#pragma unroll
      for (int e = 0; e < V; ++e)
        rotate_pair<BWD>(xv[j][0][e], xv[j][1][e], cv[0][e], cv[1][e], sv[0][e], sv[1][e],
                         ya[e], yb[e]);
      store_n<XT, V, VEC, true>(p.x, x0 + j * p.D, ya);
      store_n<XT, V, VEC, true>(p.x, x0 + j * p.D + hoff, yb);
    } else {
      float y[V];
#pragma unroll
      for (int e = 0; e < V; e += 2)
        rotate_pair<BWD>(xv[j][0][e], xv[j][0][e + 1], cv[0][e], cv[0][e + 1], sv[0][e],
                         sv[0][e + 1], y[e], y[e + 1]);
      store_n<XT, V, VEC, true>(p.x, x0 + j * p.D, y);
    }
  }
}

template <typename XT, typename CT, bool VEC, int NHL, bool CNT, bool BWD, bool HALF, bool XCH,
          bool PAD>
__global__ __launch_bounds__(kBlock) void inplace_rope_kernel(InplacePlan p) {
  // item it -> (row group r = (b, s, head group g), chunk) and the cos/sin row of r.  Two
  // loops: 32-bit indices with multiply-high division (the usual case), and plain 64-bit
  // division for huge tensors, kept apart so that the 64-bit division setup never runs in the
  // 32-bit case.
  // The grid stride is taken at entry, so that the grid size is read with the first round of
  // scalar argument loads: left in the loop, it was read in a third dependent round before
  // any lane could issue its loads (the 25 MB bf16 launch took 6.1-6.2 us that way, 5.9-6.0
  // with the stride here).
  const uint32_t stride = gridDim.x * p.block;
  asm volatile("" ::"s"(stride));
  if (p.idx32) {
    const uint32_t items = uint32_t(p.items);
    for (uint32_t it = blockIdx.x * p.block + threadIdx.x; it < items; it += stride) {
      const uint32_t r = fdiv(p.div_cpr, it);
      const uint32_t chunk = it - r * p.chunks_per_row;
      // the cos/sin row from r directly (InplacePlan::crow_a; arithmetic mod 2^32, the row
      // is below 2^31): the common layouts skip one or both divisions, and the two that
      // remain do not wait for each other
      uint32_t crow = r * p.crow_a;
      if (p.crow_b != 0) crow += fdiv(p.div_ng, r) * p.crow_b;
      if (p.crow_c != 0) crow += fdiv(p.div_ngs, r) * p.crow_c;
      // nhl * D and L are below 2^32 here: each offset is one 32 x 32 -> 64-bit product
      const uint64_t xrow = uint64_t(r) * uint32_t(p.D * NHL);
      const uint64_t crow_el = uint64_t(crow) * uint32_t(p.L);
      inplace_item<XT, CT, VEC, NHL, CNT, BWD, HALF, XCH, PAD>(p, chunk, int64_t(xrow),
                                                               int64_t(crow_el));
    }
  } else {
    const uint64_t items = uint64_t(p.items), ng = uint64_t(p.N) / NHL;
    for (uint64_t it = uint64_t(blockIdx.x) * p.block + threadIdx.x; it < items;
         it += uint64_t(gridDim.x) * p.block) {
      const uint64_t r = it / p.chunks_per_row;
      const uint64_t chunk = it - r * p.chunks_per_row;
      const uint64_t bs = r / ng;
      const uint64_t g = r - bs * ng;
      const uint64_t b = bs / uint64_t(p.S);
      const uint64_t s = bs - b * uint64_t(p.S);
      const int64_t crow = int64_t(b) * p.cb + int64_t(s) * p.cs + int64_t(g) * NHL * p.cn;
      inplace_item<XT, CT, VEC, NHL, CNT, BWD, HALF, XCH, PAD>(p, chunk, int64_t(r) * NHL * p.D,
                                                               crow * p.L);
    }
  }
}

// ============================================================================================
// K2: RoPE with a cos/sin cache ([RSCC §设计动机], rope and mrope modes, NeoX and GPT-J), tile
// form.  It serves the plans the wavefront form further below does not take: element-wise
// access (unaligned data), heads of more than 64 lanes' units, unaligned positions.
// A workgroup owns a tile of tokens.  Stage: its lanes gather each token's cos|sin row from
// the cache (mrope: element i from the position row that the stitching assigns it) and keep
// it in LDS in the cache's own element type (raised to float32 at use), so it is read from
// HBM once per token and reused by every q/k head.  Then lanes walk (token, head, unit)
// items.  NeoX: a unit is two V-element vectors, u and u + rd/(2V) of the rotated part (its
// pairs lie across the halves), or the same two-vector shape over [rd, H) copied as raw bits.
// GPT-J: a unit is one vector (its pairs lie inside it), rotated below rd and copied above.
// The units of one head are adjacent lanes.  q/k are streamed (non-temporal loads and
// stores); the first pass's loads are issued before the LDS staging so that their latency
// overlaps the position -> cache gather.
// ============================================================================================
// mrope: the position row whose section holds element i of cos/sin
// ([RSCC §mrope 模式：多模态位置编码]).
__device__ inline int mrope_section_of(const CachePlan &p, int64_t i) {
  int sec = int(i >= p.sec_end[0]) + int(i >= p.sec_end[1]);
  if (p.nsec == 4) sec += int(i >= p.sec_end[2]);
  return sec;
}

// The position row that element i (< rotaryDim/2) of the stitched cos/sin takes.  Sectioned
// (cacheMode 0): the section holding i.  Interleaved (cacheMode 1, three sections,
// [RSCC §V2 接口：cacheMode 扩展]): below 3 * mropeSection[1], elements with i % 3 == 1 come
// from row 1 and those with i % 3 == 2 from row 2; every other element from row 0.
__device__ inline int cs_row_of(const CachePlan &p, uint32_t i) {
  if (p.interleaved) {
    const uint32_t r = i % 3u;
    return (int32_t(i) < p.interleave_end && r != 0) ? int(r) : 0;
  }
  return mrope_section_of(p, i);
}

// Positions outside [0, maxSeqLen) break the contract; clamping keeps every read inside the
// cache.
__device__ inline int64_t clamp_position(const CachePlan &p, int64_t pos) {
  return pos < 0 ? 0 : (pos >= p.max_seq ? p.max_seq - 1 : pos);
}

// Word j of a 16-byte raw vector.
__device__ inline uint32_t word_of(const u32x4 &v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Where one item of a tile lives: token, q or k, head, unit, and the element offsets of its
// vectors inside the head (off_b is used by NeoX units only).
struct CacheItem {
  int64_t in_row, out_row, off_a, off_b;
  uint32_t tl, u;
  bool is_q;
};

template <bool NEOX>
__device__ inline CacheItem cache_item(const CachePlan &p, int64_t t0, uint32_t it) {
  CacheItem c;
  c.tl = fdiv(p.div_ipt, it);
  const uint32_t r = it - c.tl * p.items_per_token;
  const uint32_t h = fdiv(p.div_units, r);
  c.u = r - h * p.units;
  const int64_t t = t0 + c.tl;
  c.is_q = h < uint32_t(p.nq);
  const int64_t hh = c.is_q ? int64_t(h) : int64_t(h) - p.nq;
  c.in_row = t * (c.is_q ? p.q_stride : p.k_stride) + hh * p.H;
  c.out_row = t * ((c.is_q ? p.nq : p.nk) * p.H) + hh * p.H;
  const int64_t V = p.vec;
  if constexpr (NEOX) {
    if (c.u < p.rot_units) {
      c.off_a = int64_t(c.u) * V;
      c.off_b = p.rd / 2 + int64_t(c.u) * V;
    } else {
      const int64_t v = int64_t(c.u - p.rot_units) * V;
      c.off_a = p.rd + v;
      c.off_b = p.rd + (p.H - p.rd) / 2 + v;
    }
  } else {
    c.off_a = int64_t(c.u) * V;
    c.off_b = 0;
  }
  return c;
}

// A lane's in-flight items: only the raw vectors and the item index are kept across the
// load -> store distance (addresses are recomputed), which keeps register use low and the
// number of resident waves high.
template <typename T, int V, bool VEC, int K, int NV>
struct CacheItems {
  RawN<T, V, VEC> v[K][NV];
  uint32_t it[K];
};

constexpr uint32_t kNoItem = 0xffffffffu;

template <typename T, bool NEOX, int V, bool VEC, int K, int NV>
__device__ inline void cache_load_pass(const CachePlan &p, int64_t t0, uint32_t tile_items,
                                       uint32_t pbase, CacheItems<T, V, VEC, K, NV> &w) {
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const uint32_t it = pbase + uint32_t(k) * kCacheBlock + threadIdx.x;
    w.it[k] = it < tile_items ? it : kNoItem;
    // NeoX: a lane past the tile's end loads the tile's last item again (its lines are being
    // fetched anyway) and stores nothing.  Branch-free loads let the compiler keep far fewer
    // registers live here (62 instead of 91 VGPRs for bf16).  GPT-J keeps the branch: its
    // tiles fill whole passes, and the clamped form schedules worse for it.
    if constexpr (!NEOX)
      if (it >= tile_items) continue;
    const CacheItem c = cache_item<NEOX>(p, t0, it < tile_items ? it : tile_items - 1);
    const void *in = c.is_q ? p.q_in : p.k_in;
    load_raw<T, V, VEC, true>(in, c.in_row + c.off_a, w.v[k][0]);
    if constexpr (NV == 2) load_raw<T, V, VEC, true>(in, c.in_row + c.off_b, w.v[k][NV - 1]);
  }
}

// DIRECT: BYTES bytes of a token's cos or sin straight from its cache row (16-byte aligned
// rows: one load; otherwise element by element).
template <typename T, int BYTES>
__device__ inline Words<BYTES> cache_row_words(const T *row, bool vec) {
  Words<BYTES> r;
  if (vec) {
    load_words<BYTES, false>(row, r);
  } else {
    union {
      Words<BYTES> w;
      typename Io<T>::raw e[BYTES / int(sizeof(T))];
    } u;
    const typename Io<T>::raw *q = reinterpret_cast<const typename Io<T>::raw *>(row);
#pragma unroll
    for (int j = 0; j < BYTES / int(sizeof(T)); ++j) u.e[j] = q[j];
    r = u.w;
  }
  return r;
}

template <typename T, bool NEOX, int V, bool VEC, int K, int NV, bool DIRECT>
__device__ inline void cache_store_pass(const CachePlan &p, int64_t t0, const T *cs_tile,
                                        const CacheItems<T, V, VEC, K, NV> &w) {
  const int64_t rd = p.rd, half = rd / 2;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (w.it[k] == kNoItem) continue;
    const CacheItem c = cache_item<NEOX>(p, t0, w.it[k]);
    void *out = c.is_q ? p.q_out : p.k_out;
    if (c.u >= p.rot_units) {  // pass-through: raw bits
      store_raw<T, V, VEC, true>(out, c.out_row + c.off_a, w.v[k][0]);
      if constexpr (NV == 2) store_raw<T, V, VEC, true>(out, c.out_row + c.off_b, w.v[k][NV - 1]);
      continue;
    }
    // the token's cos|sin row: kept in LDS in the cache's own element type, or (DIRECT, rope
    // mode) read from the cache row of the token's position
    const T *cs;
    if constexpr (DIRECT)
      cs = static_cast<const T *>(p.cache) +
           clamp_position(p, p.positions[(t0 + c.tl) * p.pos_stride_tok]) * p.cache_stride;
    else
      cs = cs_tile + int64_t(c.tl) * rd;
    constexpr int PW = Io<T>::kPerWord;
    if constexpr (NEOX) {
      // [RSCC §rotate_half（GPT-NeoX style）旋转模式]: x1 = a (first half), x2 = b.  Worked one
      // 32-bit word (1 or 2 elements) of each vector at a time to keep few values live.
      const int64_t ci = int64_t(c.u) * V;
      u32x4 cw, sw;
      if constexpr (DIRECT) {
        const Words<16> cr = cache_row_words<T, 16>(cs + ci, p.cache_vec);
        const Words<16> sr = cache_row_words<T, 16>(cs + half + ci, p.cache_vec);
        cw = u32x4{cr.w[0], cr.w[1], cr.w[2], cr.w[3]};
        sw = u32x4{sr.w[0], sr.w[1], sr.w[2], sr.w[3]};
      } else {
        cw = *reinterpret_cast<const u32x4 *>(cs + ci);
        sw = *reinterpret_cast<const u32x4 *>(cs + half + ci);
      }
      RawN<T, V, VEC> oa, ob;
#pragma unroll
      for (int q = 0; q < V / PW; ++q) {
        float a[PW], b[PW], ya[PW], yb[PW], cv[PW], sv[PW];
        raw_word_to_float<T, V, VEC>(w.v[k][0], q, a);
        raw_word_to_float<T, V, VEC>(w.v[k][NV - 1], q, b);
        Io<T>::word_to_floats(word_of(cw, q), cv);
        Io<T>::word_to_floats(word_of(sw, q), sv);
#pragma unroll
        for (int e = 0; e < PW; ++e) {
          ya[e] = a[e] * cv[e] - b[e] * sv[e];
          yb[e] = b[e] * cv[e] + a[e] * sv[e];
        }
        float_to_raw_word<T, V, VEC>(ya, q, oa);
        float_to_raw_word<T, V, VEC>(yb, q, ob);
      }
      store_raw<T, V, VEC, true>(out, c.out_row + c.off_a, oa);
      store_raw<T, V, VEC, true>(out, c.out_row + c.off_b, ob);
    } else {
      // [RSCC §rotate_interleaved（GPT-J style）旋转模式]: pairs (x[2m], x[2m+1]) inside the
      // vector; vector u holds pair indices u*V/2 .. u*V/2 + V/2 - 1 (V/2 elements = 8 bytes)
      float a[V], ya[V], cv[V / 2], sv[V / 2];
      raw_to_float<T, V, VEC>(w.v[k][0], a);
      const int64_t ca = int64_t(c.u) * (V / 2);
      u32x2 cw, sw;
      if constexpr (DIRECT) {
        const Words<8> cr = cache_row_words<T, 8>(cs + ca, p.cache_vec);
        const Words<8> sr = cache_row_words<T, 8>(cs + half + ca, p.cache_vec);
        cw = u32x2{cr.w[0], cr.w[1]};
        sw = u32x2{sr.w[0], sr.w[1]};
      } else {
        cw = *reinterpret_cast<const u32x2 *>(cs + ca);
        sw = *reinterpret_cast<const u32x2 *>(cs + half + ca);
      }
      Io<T>::word_to_floats(cw.x, cv);
      Io<T>::word_to_floats(cw.y, cv + PW);
      Io<T>::word_to_floats(sw.x, sv);
      Io<T>::word_to_floats(sw.y, sv + PW);
#pragma unroll
      for (int m = 0; m < V / 2; ++m) {
        ya[2 * m] = a[2 * m] * cv[m] - a[2 * m + 1] * sv[m];
        ya[2 * m + 1] = a[2 * m + 1] * cv[m] + a[2 * m] * sv[m];
      }
      store_n<T, V, VEC, true>(out, c.out_row + c.off_a, ya);
    }
  }
}

// The position row of each element of the chunk starting at i0 (a multiple of V) in a
// 3-section plan, computed without branches.
template <int V>
__device__ inline void multi_rows(const CachePlan &p, uint32_t i0, int *row) {
  const uint32_t base = i0 % 3u;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const uint32_t e = i0 + uint32_t(j);
    uint32_t m = base + uint32_t(j % 3);
    m = m >= 3u ? m - 3u : m;  // e % 3
    const int ri = int32_t(e) < p.interleave_end ? int(m) : 0;
    const int rs = int(int32_t(e) >= p.sec_end[0]) + int(int32_t(e) >= p.sec_end[1]);
    row[j] = p.interleaved ? ri : rs;
  }
}

// MULTI: the plan's stitched cos/sin has chunks drawing on several position rows
// (CachePlan::multi_row); otherwise every staging chunk comes from one row.  DIRECT (rope mode
// with a cos|sin row too long for the LDS tile, CachePlan::cs_direct): nothing is staged; each
// item reads its cos/sin chunk from the cache row of its token's position.
template <typename T, bool NEOX, bool VEC, int K, bool MULTI, bool DIRECT>
__global__ __launch_bounds__(kCacheBlock) void cos_sin_cache_kernel(CachePlan p) {
  static_assert(!(DIRECT && MULTI), "direct cos/sin reads are a rope-mode path");
  // [tile_tokens][rd] elements of T: the gathered cos (rd/2) then sin (rd/2) of each token
  extern __shared__ u32x4 cs_lds[];
  T *cs_tile = reinterpret_cast<T *>(cs_lds);
  constexpr int V = Io<T>::kPer16;
  constexpr int NV = NEOX ? 2 : 1;  // vectors per unit
  const int64_t rd = p.rd, half = rd / 2;
  const uint32_t pass = uint32_t(kCacheBlock) * K;
  for (int64_t tile = blockIdx.x; tile < p.tiles; tile += gridDim.x) {
    // tiles [0, big_tiles) hold tile_tokens tokens, later ones a single token (tapered end)
    int64_t t0, ntok;
    if (tile < p.big_tiles) {
      t0 = tile * int64_t(p.tile_tokens);
      ntok = int64_t(p.tile_tokens);
    } else {
      t0 = p.big_tokens + (tile - p.big_tiles);
      ntok = 1;
    }
    const uint32_t tile_items = uint32_t(ntok) * p.items_per_token;

    // The position of this lane's first staging chunk is loaded before the first pass's q/k
    // loads: waiting for it does not then wait for them, and the position -> cache-row
    // chain runs while the q/k data is in flight.
    const uint32_t stage_items = uint32_t(ntok) * p.stage_chunks;
    // (Multi-row chunks load their positions at staging time: holding three positions
    // across the q/k loads costs more registers than the early load saves.)
    int64_t first_pos = 0;
    if (!MULTI && !DIRECT && threadIdx.x < stage_items) {
      const uint32_t tl = fdiv(p.div_stage, threadIdx.x);
      const uint32_t i0 = (threadIdx.x - tl * p.stage_chunks) * uint32_t(V);
      const int sec = p.mrope ? mrope_section_of(p, i0) : 0;
      first_pos = p.positions[sec * p.pos_stride_row + (t0 + tl) * p.pos_stride_tok];
    }

    CacheItems<T, V, VEC, K, NV> w;
    cache_load_pass<T, NEOX, V, VEC, K, NV>(p, t0, tile_items, 0, w);

    // ---- stage the tile's cos|sin rows in LDS: gather, split, stitch ----
    // Values stay in the cache's element type (bits copied, raised to float32 at use).
    // Chunks that draw on several position rows (MULTI, 16-byte cache rows): one lane per
    // (chunk, row).  It loads its row's position and 16-byte cos and sin chunks, and writes
    // the elements that the stitching assigns to that row.  A row the chunk does not use
    // loads the row of the chunk's first element instead (lines already being fetched) and
    // writes nothing.  Loads are unconditional: loads under divergent branches make the
    // compiler wait for every outstanding load at each join.
    bool staged = DIRECT;
    if constexpr (MULTI) {
      if (p.cache_vec) {
        staged = true;
        using R = typename Io<T>::raw;
        for (uint32_t idx = threadIdx.x; idx < stage_items * 3u; idx += kCacheBlock) {
          const uint32_t chunk = idx / 3u, row = idx - chunk * 3u;
          const uint32_t tl = fdiv(p.div_stage, chunk);
          const uint32_t i0 = (chunk - tl * p.stage_chunks) * uint32_t(V);
          int rows[V];
          multi_rows<V>(p, i0, rows);
          bool used = false;
#pragma unroll
          for (int j = 0; j < V; ++j) used |= rows[j] == int(row);
          const int64_t rsel = used ? int64_t(row) : int64_t(rows[0]);
          const int64_t pos = p.positions[rsel * p.pos_stride_row + (t0 + tl) * p.pos_stride_tok];
          const T *src =
              static_cast<const T *>(p.cache) + clamp_position(p, pos) * p.cache_stride + i0;
          union Chunk {
            u32x4 v;
            R e[V];
          };
          Chunk c, sn;
          c.v = ld16<false>(src);
          sn.v = ld16<false>(src + half);
          R *dst = reinterpret_cast<R *>(cs_tile + int64_t(tl) * rd + i0);
#pragma unroll
          for (int j = 0; j < V; ++j)
            if (rows[j] == int(row)) {
              dst[j] = c.e[j];
              dst[half + j] = sn.e[j];
            }
        }
      }
    }
    // Otherwise one lane per V-element chunk of a token's cos half (and the matching sin
    // chunk): a chunk drawn from one position row (always, in rope mode) is copied as 16-byte
    // vectors; an unaligned cache is gathered element by element.
    for (uint32_t idx = threadIdx.x; !staged && idx < stage_items; idx += kCacheBlock) {
      const uint32_t tl = fdiv(p.div_stage, idx);
      const uint32_t i0 = (idx - tl * p.stage_chunks) * uint32_t(V);
      const int64_t tok = (t0 + tl) * p.pos_stride_tok;
      T *dst = cs_tile + int64_t(tl) * rd + i0;
      using R = typename Io<T>::raw;
      if (!p.cache_vec) {  // rare: kept rolled so it does not raise the register count
#pragma unroll 1
        for (int j = 0; j < V; ++j) {
          const int r = p.mrope ? cs_row_of(p, i0 + uint32_t(j)) : 0;
          const int64_t row = clamp_position(p, p.positions[r * p.pos_stride_row + tok]) *
                              p.cache_stride;
          const R *src = static_cast<const R *>(p.cache) + row + i0 + j;
          reinterpret_cast<R *>(dst)[j] = src[0];
          reinterpret_cast<R *>(dst + half)[j] = src[half];
        }
      } else {
        const int sec = p.mrope ? mrope_section_of(p, i0) : 0;
        const int64_t pos =
            idx == threadIdx.x ? first_pos : p.positions[sec * p.pos_stride_row + tok];
        const T *src =
            static_cast<const T *>(p.cache) + clamp_position(p, pos) * p.cache_stride + i0;
        *reinterpret_cast<u32x4 *>(dst) = ld16<false>(src);
        *reinterpret_cast<u32x4 *>(dst + half) = ld16<false>(src + half);
      }
    }
    if constexpr (!DIRECT) __syncthreads();

    // ---- rotate the first rd of every q head then k head, copy the rest ----
    for (uint32_t pbase = 0;;) {
      cache_store_pass<T, NEOX, V, VEC, K, NV, DIRECT>(p, t0, cs_tile, w);
      pbase += pass;
      if (pbase >= tile_items) break;
      cache_load_pass<T, NEOX, V, VEC, K, NV>(p, t0, tile_items, pbase, w);
    }
    if constexpr (!DIRECT) __syncthreads();  // the LDS tile is rewritten by the next tile
  }
}

// ============================================================================================
// K2, wavefront form (the plans it covers: 16-byte q/k and cache access, a head's units on at
// most 64 lanes, 8-byte aligned positions).  The same operation as cos_sin_cache_kernel, with
// one wavefront per (token, group of heads) and no LDS and no barrier.  Lane l owns unit
// u = l % units of head l / units in each of K rows of wave_hpw heads (K: the plan's
// wave_rows, so that every lane carries two 16-byte q/k vectors), so its cos|sin chunk (NeoX:
// the V elements u*V...; GPT-J: the V/2 pair indices u*V/2...) is the same for all of its items
// and is read straight from the token's cache row; the lanes of one unit read the same bytes,
// which the caches serve.  The token's positions are wave-uniform and are read through the
// scalar cache, so waiting for them does not wait for the q/k loads in flight.
// ============================================================================================
typedef const __attribute__((address_space(4))) int64_t const_i64;

// Output rows of the wavefront kernel as buffer ranges.  Its q/k stores go out as buffer stores
// with the device-scope and streaming cache bits (sc1 | nt): on MI355X those copy 0.4-2.5%
// faster than the plain non-temporal global stores of the same bytes, where nt alone is no
// faster and sc1 alone slower.  A range is one token's q (or k) output row, below 2^31 bytes
// on this path, so every offset is a 32-bit byte offset inside it.
constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, no swizzle, no index stride
constexpr int kStoreSc1Nt = 16 | 2;     // cache-policy bits of the store: sc1 | nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_range(void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, int(bytes), kRsrcWord3);
}

template <typename T, int V>
__device__ __forceinline__ void row_store(__amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rk,
                                          bool is_q, int64_t elem, const RawN<T, V, true> &r) {
  const int off = int(elem * int64_t(sizeof(T)));
  if (is_q) __builtin_amdgcn_raw_buffer_store_b128(r.v[0], rq, off, 0, kStoreSc1Nt);
  else __builtin_amdgcn_raw_buffer_store_b128(r.v[0], rk, off, 0, kStoreSc1Nt);
}

// The lane's cos (or sin) chunk as raw elements of T.
template <typename T, int CB>
union CsChunk {
  Words<CB> w;
  typename Io<T>::raw e[CB / int(sizeof(T))];
};

// XCH (NeoX with rotaryDim <= headSize/2): lane u's first access takes vector u of the head
// and its second vector units + u, so each access instruction covers whole lines of the heads
// (with the two-vector units, a partial rotaryDim left every access half or a quarter of each
// line it touched).  All rotated vectors are then in the first access, lanes 0 .. 2R-1
// (R = rotated units); the pair partner of vector u is vector u + R or u - R, which its own
// lane holds, and is read from there with ds_bpermute.  Each lane rotates its own vector.
// LIN (NeoX): a unit is one vector, as in GPT-J, so a head's vectors lie on consecutive lanes
// and each access covers whole heads; the pair partner (R vectors away, R = rotaryDim/(2V))
// is read from its lane with ds_bpermute, as in XCH.  In both, outside multi-row stitching,
// the two lanes of a pair also share the gather of their cos|sin chunk (one 16-byte load each,
// swapped over the same exchange).  Against both halves gathered per lane: LIN rope-mode shapes
// 4-7% faster, XCH 1% (4% at 512 tokens), three-section mrope within noise.
// NR: position rows read per token: 1 in rope mode (no section table), else the mrope
// section count (3 or 4; multi-row stitching has 3).
// WB: lanes per workgroup (the plan's wave_block).  SR: the token's cos|sin row is read with
// scalar loads (the plan's wave_scalar_row: GPT-J rope mode, 128-byte rows).
template <typename T, bool NEOX, bool MULTI, bool XCH, bool LIN, int NR, int K, int WB, bool SR>
__global__ __launch_bounds__(WB) void cos_sin_cache_wave_kernel(CachePlan p) {
  static_assert(!(XCH || LIN) || NEOX, "the lane exchange is a NeoX layout");
  static_assert(!(XCH && LIN), "one layout at a time");
  static_assert(NR == 1 || NR == 3 || NR == 4, "rope mode or an mrope section count");
  static_assert(!MULTI || NR == 3, "multi-row stitching reads three rows");
  constexpr bool MR = NR > 1;
  constexpr bool EXCH = XCH || LIN;
  // One-vector units (GPT-J, LIN): the wavefront issues its loads at raised priority and drops
  // back once they are all out (below), so that wavefronts starting up get their loads in ahead
  // of the rotation and stores of older ones.  GPT-J in one-wavefront workgroups: the 1 GiB f16
  // workload 1.8% faster, 64 and 512 tokens 5-7%, other shapes within 2% either way; LIN 6%
  // faster.  The pair units (3%) and the exchange layout (4-5%) were slower with it.
  constexpr bool PRIO = !NEOX || LIN;
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(3);  // rotated vectors pair across lanes
  constexpr int V = Io<T>::kPer16;
  constexpr int NV = NEOX && !LIN ? 2 : 1;  // vectors per unit
  constexpr int C = NEOX ? V : V / 2;  // cos (and sin) elements of the lane's chunk
  constexpr int CB = C * int(sizeof(T));  // 16 bytes (NeoX) or 8 (GPT-J)
  constexpr int PW = Io<T>::kPerWord;
  const uint32_t lane = __lane_id();
  const uint32_t lanes_per_head = LIN ? 2 * p.units : p.units;
  const uint32_t hsub = lane / lanes_per_head;
  const uint32_t u = lane - hsub * lanes_per_head;
  const bool lane_on = hsub < p.wave_hpw;  // lanes past the last whole head are idle
  const uint32_t hs = lane_on ? hsub : 0;   // (idle lanes load like the first head row)
  const uint32_t R = p.rot_units;
  // rot: the lane's (first) vector is rotated; cu: the cos|sin chunk it uses
  const bool rot = EXCH ? u < 2 * R : u < R;
  const uint32_t cu = !rot ? 0 : (EXCH && u >= R) ? u - R : u;
  const int64_t rd = p.rd, half = rd / 2, nh = p.nq + p.nk;
  const int64_t i0 = int64_t(cu) * C;  // first cos element of the lane's chunk
  // XCH: the lane holding the pair partners of this lane's first vector (ds_bpermute address)
  const int xaddr =
      int(((EXCH && rot && lane_on) ? lane - u + (u < R ? u + R : u - R) : lane) << 2);
  // element offsets of the lane's vectors inside a head, the same for each of its items
  int64_t off_a, off_b = 0;
  if constexpr (XCH) {
    off_a = int64_t(u) * V;
    off_b = p.H / 2 + int64_t(u) * V;
  } else if constexpr (LIN) {
    off_a = int64_t(u) * V;
  } else if constexpr (NEOX) {
    if (rot) {
      off_a = int64_t(u) * V;
      off_b = half + int64_t(u) * V;
    } else {
      const int64_t w = int64_t(u - p.rot_units) * V;
      off_a = rd + w;
      off_b = rd + (p.H - rd) / 2 + w;
    }
  } else {
    off_a = int64_t(u) * V;
  }
  // MULTI: the position row of element j of the chunk in bits 2j, 2j+1 (one register instead
  // of C); otherwise the one row of the whole chunk
  uint32_t rmask = 0;
  int sec = 0;
  if constexpr (MULTI) {
    int rows[C];
    multi_rows<C>(p, uint32_t(i0), rows);
#pragma unroll
    for (int j = 0; j < C; ++j) rmask |= uint32_t(rows[j]) << (2 * j);
  } else if constexpr (MR) {
    sec = mrope_section_of(p, i0);
  }
  const_i64 *pos_s = reinterpret_cast<const_i64 *>(reinterpret_cast<uintptr_t>(p.positions));
  // Offsets of the NR position rows: unconditional loads, which the compiler keeps in flight
  // across the q/k loads (loads under a branch were waited for before the q/k loads went
  // out).  Exactly the rows the plan has: with four loads of one address in rope mode, the
  // rope NeoX bf16 workload took 29.7-29.9 us, 28.8-28.9 with one.
  int64_t roff[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) roff[r] = int64_t(r) * p.pos_stride_row;
  constexpr uint32_t kWpb = WB / 64;
  for (uint32_t gw = __builtin_amdgcn_readfirstlane(blockIdx.x * kWpb + threadIdx.x / 64);
       gw < uint32_t(p.waves); gw += gridDim.x * kWpb) {
    const uint32_t t32 = fdiv(p.div_wpt, gw);
    const int64_t t = t32;
    const int64_t hbase = int64_t(gw - t32 * p.wave_wpt) * p.wave_heads + hs;
    const int64_t qrow = p.nq * p.H, krow = p.nk * p.H;  // elements of a token's output rows
    const __amdgpu_buffer_rsrc_t rq =
        row_range(static_cast<T *>(p.q_out) + t * qrow, qrow * int64_t(sizeof(T)));
    const __amdgpu_buffer_rsrc_t rk =
        row_range(static_cast<T *>(p.k_out) + t * krow, krow * int64_t(sizeof(T)));
    // the token's position rows (wave-uniform scalar loads; they go out with the q/k loads
    // below and are waited for only after those, see the asm statement)
    int64_t prow[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) prow[r] = pos_s[roff[r] + t * p.pos_stride_tok];
    // q/k loads of every item (a lane past the last head loads the last head again and
    // stores nothing)
    RawN<T, V, true> v[K][NV];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      int64_t h = hbase + int64_t(k) * p.wave_hpw;
      h = h < nh ? h : nh - 1;
      const bool is_q = h < p.nq;
      const int64_t in_row = t * (is_q ? p.q_stride : p.k_stride) + (is_q ? h : h - p.nq) * p.H;
      const void *in = is_q ? p.q_in : p.k_in;
      load_raw<T, V, true, true>(in, in_row + off_a, v[k][0]);
      if constexpr (NV == 2) load_raw<T, V, true, true>(in, in_row + off_b, v[k][NV - 1]);
    }
    // All four positions are needed here, after the q/k loads went out: otherwise the compiler
    // moves each scalar load under the per-lane row choice below and waits for them in turn.
    if constexpr (NR == 4) asm volatile("" ::"s"(prow[0]), "s"(prow[1]), "s"(prow[2]), "s"(prow[3]));
    else if constexpr (NR == 3) asm volatile("" ::"s"(prow[0]), "s"(prow[1]), "s"(prow[2]));
    else asm volatile("" ::"s"(prow[0]));
    // the lane's cos and sin chunks: gather, split, stitch
    CsChunk<T, CB> cw, sw;
    if constexpr (MULTI) {
      CsChunk<T, CB> cr[3], sr[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const T *row = static_cast<const T *>(p.cache) + clamp_position(p, prow[r]) * p.cache_stride;
        load_words<CB, false>(row + i0, cr[r].w);
        load_words<CB, false>(row + half + i0, sr[r].w);
      }
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const uint32_t r = (rmask >> (2 * j)) & 3u;
        cw.e[j] = r == 0 ? cr[0].e[j] : r == 1 ? cr[1].e[j] : cr[2].e[j];
        sw.e[j] = r == 0 ? sr[0].e[j] : r == 1 ? sr[1].e[j] : sr[2].e[j];
      }
    } else {
      int64_t pos = prow[0];
      if constexpr (NR == 3) pos = sec == 0 ? prow[0] : sec == 1 ? prow[1] : prow[2];
      if constexpr (NR == 4)
        pos = sec == 0 ? prow[0] : sec == 1 ? prow[1] : sec == 2 ? prow[2] : prow[3];
      const T *row = static_cast<const T *>(p.cache) + clamp_position(p, pos) * p.cache_stride;
      if constexpr (SR) {
        static_assert(!NEOX && NR == 1 && CB == 8, "GPT-J rope mode, 8-byte chunks");
        // The whole 128-byte row in scalar registers (two 64-byte scalar loads: the row is
        // wave-uniform): cos chunk c is words 2c, 2c + 1 and its sin chunk words 16 + 2c,
        // 17 + 2c, c < 8; each lane selects its own chunk cu.  The empty asm keeps the words in
        // SGPRs (otherwise the compiler turns the selection back into per-lane vector loads).
        typedef const __attribute__((address_space(4))) uint32_t const_u32;
        const_u32 *rw = reinterpret_cast<const_u32 *>(reinterpret_cast<uintptr_t>(row));
        uint32_t w[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) w[i] = rw[i];
#pragma unroll
        for (int i = 0; i < 32; ++i) asm volatile("" : "+s"(w[i]));
        // word `first` of chunk cu: a three-level select on the bits of cu
        const bool b0 = (cu & 1u) != 0, b1 = (cu & 2u) != 0, b2 = (cu & 4u) != 0;
        const auto pick = [&](int first) {
          const uint32_t l0 = b0 ? w[first + 2] : w[first];
          const uint32_t l1 = b0 ? w[first + 6] : w[first + 4];
          const uint32_t l2 = b0 ? w[first + 10] : w[first + 8];
          const uint32_t l3 = b0 ? w[first + 14] : w[first + 12];
          return b2 ? (b1 ? l3 : l2) : (b1 ? l1 : l0);
        };
        cw.w.w[0] = pick(0);
        cw.w.w[1] = pick(1);
        sw.w.w[0] = pick(16);
        sw.w.w[1] = pick(17);
        // Every row's q/k data is needed here, before any store, as the vector cos/sin loads
        // make the other path wait: waiting only for the first row, the compiler had the
        // second row wait for the first row's store as well (the counter is in order).
#pragma unroll
        for (int k = 0; k < K; ++k) asm volatile("" ::"v"(v[k][0].v[0].x));
      } else if constexpr (EXCH) {
        // the pair's two lanes share one chunk: the x1 lane gathers its cos half, the x2 lane
        // its sin half, and each takes the other half from its partner below
        load_words<CB, false>(row + (u < R ? int64_t(0) : half) + i0, cw.w);
      } else {
        load_words<CB, false>(row + i0, cw.w);
        load_words<CB, false>(row + half + i0, sw.w);
      }
    }
    // Every load of the item is out: keep the compiler from moving work that waits for the
    // q/k data above the cos/sin loads.  Left to itself it waited for the first q/k vector
    // between the cos and the sin load of NeoX pair units, which serialized two round trips:
    // with one head row per lane the rope NeoX workload took 30.4 us without this barrier and
    // 28.7 us with it (29.6 us with two rows).
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    if constexpr (EXCH && !MULTI) {
      // XCH, LIN: swap the gathered halves with the pair partner (idle and copy-only lanes read
      // their own registers)
      const bool x1 = u < R;
#pragma unroll
      for (int q = 0; q < CB / 4; ++q) {
        const uint32_t mine = cw.w.w[q];
        const uint32_t other = uint32_t(__builtin_amdgcn_ds_bpermute(xaddr, int(mine)));
        cw.w.w[q] = x1 ? mine : other;
        sw.w.w[q] = x1 ? other : mine;
      }
    }
    // rotate the first rd of every head, copy the rest as raw bits
#pragma unroll
    for (int k = 0; k < K; ++k) {
      // XCH: every lane takes part in the exchange before any lane branches off
      RawN<T, V, true> xp;
      if constexpr (EXCH) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = word_of(v[k][0].v[0], q);
          const uint32_t r = uint32_t(__builtin_amdgcn_ds_bpermute(xaddr, int(w)));
          if (q == 0) xp.v[0].x = r;
          else if (q == 1) xp.v[0].y = r;
          else if (q == 2) xp.v[0].z = r;
          else xp.v[0].w = r;
        }
      }
      const int64_t h = hbase + int64_t(k) * p.wave_hpw;
      if (!lane_on || h >= nh) continue;
      const bool is_q = h < p.nq;
      const int64_t out_row = (is_q ? h : h - p.nq) * p.H;  // inside the token's output row
      if constexpr (EXCH) {
        if constexpr (XCH) row_store<T, V>(rq, rk, is_q, out_row + off_b, v[k][NV - 1]);
        if (!rot) {
          row_store<T, V>(rq, rk, is_q, out_row + off_a, v[k][0]);
          continue;
        }
        // [RSCC §rotate_half（GPT-NeoX style）旋转模式]: the x1 lane (u < R) writes
        // x1*cos - x2*sin, the x2 lane x2*cos + x1*sin; "a" is the lane's own element, "b" its
        // partner's
        const bool x1_lane = u < R;
        RawN<T, V, true> oa;
#pragma unroll
        for (int q = 0; q < V / PW; ++q) {
          float a[PW], b[PW], y[PW], cv[PW], sv[PW];
          raw_word_to_float<T, V, true>(v[k][0], q, a);
          raw_word_to_float<T, V, true>(xp, q, b);
          Io<T>::word_to_floats(cw.w.w[q], cv);
          Io<T>::word_to_floats(sw.w.w[q], sv);
#pragma unroll
          for (int e = 0; e < PW; ++e) {
            const float pr = a[e] * cv[e];
            const float qr = b[e] * sv[e];
            y[e] = x1_lane ? pr - qr : pr + qr;
          }
          float_to_raw_word<T, V, true>(y, q, oa);
        }
        row_store<T, V>(rq, rk, is_q, out_row + off_a, oa);
        continue;
      }
      if (!rot) {
        row_store<T, V>(rq, rk, is_q, out_row + off_a, v[k][0]);
        if constexpr (NV == 2) row_store<T, V>(rq, rk, is_q, out_row + off_b, v[k][NV - 1]);
        continue;
      }
      if constexpr (NEOX) {
        // [RSCC §rotate_half（GPT-NeoX style）旋转模式]: x1 = a (first half), x2 = b
        RawN<T, V, true> oa, ob;
#pragma unroll
        for (int q = 0; q < V / PW; ++q) {
          float a[PW], b[PW], ya[PW], yb[PW], cv[PW], sv[PW];
          raw_word_to_float<T, V, true>(v[k][0], q, a);
          raw_word_to_float<T, V, true>(v[k][NV - 1], q, b);
          Io<T>::word_to_floats(cw.w.w[q], cv);
          Io<T>::word_to_floats(sw.w.w[q], sv);
#pragma unroll
          for (int e = 0; e < PW; ++e) {
            ya[e] = a[e] * cv[e] - b[e] * sv[e];
            yb[e] = b[e] * cv[e] + a[e] * sv[e];
          }
          float_to_raw_word<T, V, true>(ya, q, oa);
          float_to_raw_word<T, V, true>(yb, q, ob);
        }
        row_store<T, V>(rq, rk, is_q, out_row + off_a, oa);
        row_store<T, V>(rq, rk, is_q, out_row + off_b, ob);
      } else {
        // [RSCC §rotate_interleaved（GPT-J style）旋转模式]: pairs (x[2m], x[2m+1]) inside the
        // vector, with cos/sin entry m of the lane's chunk
        float a[V], ya[V], cv[C], sv[C];
        raw_to_float<T, V, true>(v[k][0], a);
        words_to_floats<T, C>(cw.w, cv);
        words_to_floats<T, C>(sw.w, sv);
#pragma unroll
        for (int m = 0; m < C; ++m) {
          ya[2 * m] = a[2 * m] * cv[m] - a[2 * m + 1] * sv[m];
          ya[2 * m + 1] = a[2 * m + 1] * cv[m] + a[2 * m] * sv[m];
        }
        RawN<T, V, true> oy;
#pragma unroll
        for (int q = 0; q < V / PW; ++q) float_to_raw_word<T, V, true>(ya + q * PW, q, oy);
        row_store<T, V>(rq, rk, is_q, out_row + off_a, oy);
      }
    }
  }
}

// ---- launch helpers -------------------------------------------------------------------------


thread_local std::string g_last_error;

int launch(const void *fn, int64_t blocks, int threads, size_t lds, void *stream, void *plan) {
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  void *args[] = {plan};
  hipError_t e = hipLaunchKernel(fn, dim3(uint32_t(blocks)), dim3(uint32_t(threads)), args, lds,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = std::string("kernel launch failed: ") + hipGetErrorString(e);
    return ROPE_ERR_RUNTIME;
  }
  return ROPE_OK;
}

template <typename XT, typename CT, bool BWD, bool HALF, bool XCH, bool PAD>
const void *pick_inplace_vec(const InplacePlan &p) {
#define ROPE_K1(NHL, CNT) \
  reinterpret_cast<const void *>(                                                       \
      &inplace_rope_kernel<XT, CT, true, NHL, CNT, BWD, HALF, XCH, PAD>)
  // Only the heads-per-lane counts a plan can choose are built: a lane's x bytes stay at 32
  // or less (x bytes per head: V elements, twice that when a lane owns both halves).
  constexpr int kV = 16 / int(sizeof(XT) > sizeof(CT) ? sizeof(XT) : sizeof(CT));
  constexpr int kXBytes = kV * int(sizeof(XT)) * (HALF && !XCH ? 2 : 1);
  if (p.nhl == 1) return p.cos_stream ? ROPE_K1(1, true) : ROPE_K1(1, false);
  if constexpr (2 * kXBytes <= 32)
    if (p.nhl == 2) return p.cos_stream ? ROPE_K1(2, true) : ROPE_K1(2, false);
  if constexpr (4 * kXBytes <= 32)
    if (p.nhl == 4) return p.cos_stream ? ROPE_K1(4, true) : ROPE_K1(4, false);
  return nullptr;  // no plan asks for this (the host plan check covers every plan shape)
#undef ROPE_K1
}

template <typename XT, typename CT, bool BWD, bool HALF>
const void *pick_inplace(const InplacePlan &p) {
  if (!p.vector_io)
    return reinterpret_cast<const void *>(
        &inplace_rope_kernel<XT, CT, false, 1, false, BWD, HALF, false, false>);
  if constexpr (HALF)
    if (p.xch != 0)
      return p.xch_cph == p.xch ? pick_inplace_vec<XT, CT, BWD, true, true, false>(p)
                                : pick_inplace_vec<XT, CT, BWD, true, true, true>(p);
  return pick_inplace_vec<XT, CT, BWD, HALF, false, false>(p);
}

template <bool BWD, bool HALF>
const void *pick_inplace_dtype(const InplacePlan &p) {
  if (p.xdt == ROPE_F32) return pick_inplace<float, float, BWD, HALF>(p);
  if (p.xdt == ROPE_F16)
    return p.cdt == ROPE_F32 ? pick_inplace<_Float16, float, BWD, HALF>(p)
                             : pick_inplace<_Float16, _Float16, BWD, HALF>(p);
  return p.cdt == ROPE_F32 ? pick_inplace<__bf16, float, BWD, HALF>(p)
                           : pick_inplace<__bf16, __bf16, BWD, HALF>(p);
}

template <typename T, bool MULTI, bool DIRECT>
const void *pick_cache_rows(bool neox, bool vec) {
  constexpr int KN = kNeoxItemsPerLane, KJ = kGptjItemsPerLane;
#define ROPE_K2(NX, VE, KK) \
  reinterpret_cast<const void *>(&cos_sin_cache_kernel<T, NX, VE, KK, MULTI, DIRECT>)
  if (neox) return vec ? ROPE_K2(true, true, KN) : ROPE_K2(true, false, KN);
  return vec ? ROPE_K2(false, true, KJ) : ROPE_K2(false, false, KJ);
#undef ROPE_K2
}

// The wavefront kernel of a layout, with the head rows per lane the plan chose (a plan that
// disagrees gets no kernel).
template <typename T, bool NX, bool XC, bool LI>
const void *pick_wave(const CachePlan &p) {
  constexpr int KP = NX && !XC && !LI ? int(kWaveRowsPairUnits) : int(kWaveRowsVectorUnits);
  constexpr int KM = int(kWaveRowsVectorUnits);  // multi-row stitching
  constexpr int WB = NX ? kWaveBlockNeox : kWaveBlockGptj;
  if (p.wave_block != uint32_t(WB)) return nullptr;
  if (p.wave_scalar_row && (NX || p.mrope || p.rd * int64_t(sizeof(T)) != kScalarRowBytes))
    return nullptr;
#define ROPE_KW(MU, NR, KK, SR) \
  reinterpret_cast<const void *>(&cos_sin_cache_wave_kernel<T, NX, MU, XC, LI, NR, KK, WB, SR>)
  if (p.multi_row)
    return p.wave_rows == uint32_t(KM) && p.nsec == 3 ? ROPE_KW(true, 3, KM, false) : nullptr;
  if (p.wave_rows != uint32_t(KP)) return nullptr;
  if (!p.mrope) {
    if constexpr (!NX)
      if (p.wave_scalar_row) return ROPE_KW(false, 1, KP, true);
    return ROPE_KW(false, 1, KP, false);
  }
  return p.nsec == 3   ? ROPE_KW(false, 3, KP, false)
         : p.nsec == 4 ? ROPE_KW(false, 4, KP, false)
                       : nullptr;
#undef ROPE_KW
}

template <typename T>
const void *pick_cache(const CachePlan &p) {
  if (p.wave) {
    if (p.neox && p.wave_lin) return pick_wave<T, true, false, true>(p);
    if (p.neox && p.wave_xch) return pick_wave<T, true, true, false>(p);
    if (p.neox) return pick_wave<T, true, false, false>(p);
    return pick_wave<T, false, false, false>(p);
  }
  if (p.cs_direct) return pick_cache_rows<T, false, true>(p.neox, p.vector_io);
  return p.multi_row ? pick_cache_rows<T, true, false>(p.neox, p.vector_io)
                     : pick_cache_rows<T, false, false>(p.neox, p.vector_io);
}

}  // namespace
}  // namespace ropeamd

using namespace ropeamd;

#define ROPE_API extern "C" __attribute__((visibility("default")))

namespace ropeamd {
namespace {

int run_inplace(const rope_tensor *x, const rope_tensor *cos, const rope_tensor *sin,
                int64_t rotary_mode, const int64_t *partial_slice, int64_t partial_slice_len,
                void *stream, bool backward) {
  InplacePlan plan;
  std::string err;
  const int st = plan_inplace(x, cos, sin, rotary_mode, partial_slice, partial_slice_len, &plan,
                              &err);
  if (st != ROPE_OK) {
    g_last_error = err;
    return st;
  }
  g_last_error.clear();
  if (plan.noop) return ROPE_OK;
  const void *fn = plan.half ? (backward ? pick_inplace_dtype<true, true>(plan)
                                         : pick_inplace_dtype<false, true>(plan))
                            : (backward ? pick_inplace_dtype<true, false>(plan)
                                        : pick_inplace_dtype<false, false>(plan));
  if (fn == nullptr) {
    g_last_error = "internal: no kernel for this plan";
    return ROPE_ERR_RUNTIME;
  }
  return launch(fn, (plan.items + plan.block - 1) / plan.block, int(plan.block), 0, stream, &plan);
}

}  // namespace
}  // namespace ropeamd

ROPE_API int rope_partial_inplace(const rope_tensor *x, const rope_tensor *cos,
                                  const rope_tensor *sin, int64_t rotary_mode,
                                  const int64_t *partial_slice, int64_t partial_slice_len,
                                  void *stream) {
  return run_inplace(x, cos, sin, rotary_mode, partial_slice, partial_slice_len, stream, false);
}

ROPE_API int rope_partial_inplace_backward(const rope_tensor *g, const rope_tensor *cos,
                                           const rope_tensor *sin, int64_t rotary_mode,
                                           const int64_t *partial_slice,
                                           int64_t partial_slice_len, void *stream) {
  return run_inplace(g, cos, sin, rotary_mode, partial_slice, partial_slice_len, stream, true);
}

ROPE_API int rope_with_cos_sin_cache_v2(const rope_tensor *positions, const rope_tensor *query_in,
                                        const rope_tensor *key_in,
                                        const rope_tensor *cos_sin_cache,
                                        const int64_t *mrope_section, int64_t mrope_section_len,
                                        int64_t head_size, int is_neox_style, int64_t cache_mode,
                                        const rope_tensor *query_out, const rope_tensor *key_out,
                                        void *stream) {
  CachePlan plan;
  std::string err;
  const int st = plan_cache(positions, query_in, key_in, cos_sin_cache, mrope_section,
                            mrope_section_len, head_size, is_neox_style, cache_mode, query_out,
                            key_out, &plan, &err);
  if (st != ROPE_OK) {
    g_last_error = err;
    return st;
  }
  g_last_error.clear();
  const void *fn = plan.dt == ROPE_F32   ? pick_cache<float>(plan)
                   : plan.dt == ROPE_F16 ? pick_cache<_Float16>(plan)
                                         : pick_cache<__bf16>(plan);
  if (fn == nullptr) {
    g_last_error = "internal: no kernel for this plan";
    return ROPE_ERR_RUNTIME;
  }
  if (plan.wave) {
    const int64_t wpb = plan.wave_block / 64;  // wavefronts per workgroup
    return launch(fn, (plan.waves + wpb - 1) / wpb, int(plan.wave_block), 0, stream, &plan);
  }
  const size_t esize = plan.dt == ROPE_F32 ? 4 : 2;
  const size_t lds = plan.cs_direct ? 0 : size_t(plan.tile_tokens) * size_t(plan.rd) * esize;
  return launch(fn, plan.tiles, kCacheBlock, lds, stream, &plan);
}

ROPE_API int rope_with_cos_sin_cache(const rope_tensor *positions, const rope_tensor *query_in,
                                     const rope_tensor *key_in, const rope_tensor *cos_sin_cache,
                                     const int64_t *mrope_section, int64_t mrope_section_len,
                                     int64_t head_size, int is_neox_style,
                                     const rope_tensor *query_out, const rope_tensor *key_out,
                                     void *stream) {
  return rope_with_cos_sin_cache_v2(positions, query_in, key_in, cos_sin_cache, mrope_section,
                                    mrope_section_len, head_size, is_neox_style, 0, query_out,
                                    key_out, stream);
}

ROPE_API const char *rope_last_error(void) { return g_last_error.c_str(); }
