// rope_kernels.hip -- gfx950 (MI355X) kernels and C-ABI entry points of librope_amd.so.
//
// Both operations are elementwise rotations of (pairs of) activations by cos/sin values: a
// few flops per 4+ bytes moved, so they are bound by HBM bandwidth.  There is no contraction
// here (no MFMA); the kernels are built around wide, coalesced 16-byte accesses, every pair
// of a rotation held in one lane's registers (no cross-lane exchange is needed), float32
// arithmetic with one rounding per product and per sum, and one rounding to the storage type.
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
  using raw = uint32_t;
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
  using raw = uint16_t;
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
  using raw = uint16_t;
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

// N consecutive elements starting at element `i` of `p`, as float32.  VEC: the address is
// 16-byte aligned and N * sizeof(T) is a multiple of 16, so whole 16-byte loads are used.
template <typename T, int N, bool VEC>
__device__ inline void load_n(const void *p, int64_t i, float *f) {
  if constexpr (VEC) {
    const uint4 *q = reinterpret_cast<const uint4 *>(static_cast<const T *>(p) + i);
#pragma unroll
    for (int c = 0; c < N / Io<T>::kPer16; ++c) Io<T>::unpack(q[c], f + c * Io<T>::kPer16);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) f[e] = Io<T>::load1(p, i + e);
  }
}

template <typename T, int N, bool VEC>
__device__ inline void store_n(void *p, int64_t i, const float *f) {
  if constexpr (VEC) {
    uint4 *q = reinterpret_cast<uint4 *>(static_cast<T *>(p) + i);
#pragma unroll
    for (int c = 0; c < N / Io<T>::kPer16; ++c) q[c] = Io<T>::pack(f + c * Io<T>::kPer16);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) Io<T>::store1(p, i + e, f[e]);
  }
}

// Raw copy of N elements (pass-through data is moved as bits, never converted).
template <typename T, int N, bool VEC>
struct RawN {
  uint4 v[VEC ? (N * int(sizeof(T)) + 15) / 16 : 1];
  typename Io<T>::raw e[VEC ? 1 : N];
};

template <typename T, int N, bool VEC>
__device__ inline void load_raw(const void *p, int64_t i, RawN<T, N, VEC> &r) {
  if constexpr (VEC) {
    const uint4 *q = reinterpret_cast<const uint4 *>(static_cast<const T *>(p) + i);
#pragma unroll
    for (int c = 0; c < (N * int(sizeof(T))) / 16; ++c) r.v[c] = q[c];
  } else {
    const typename Io<T>::raw *q = static_cast<const typename Io<T>::raw *>(p) + i;
#pragma unroll
    for (int e = 0; e < N; ++e) r.e[e] = q[e];
  }
}

template <typename T, int N, bool VEC>
__device__ inline void store_raw(void *p, int64_t i, const RawN<T, N, VEC> &r) {
  if constexpr (VEC) {
    uint4 *q = reinterpret_cast<uint4 *>(static_cast<T *>(p) + i);
#pragma unroll
    for (int c = 0; c < (N * int(sizeof(T))) / 16; ++c) q[c] = r.v[c];
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
    for (int c = 0; c < (N * int(sizeof(T))) / 16; ++c) Io<T>::unpack(r.v[c], f + c * Io<T>::kPer16);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) f[e] = Io<T>::from_raw(r.e[e]);
  }
}

__device__ inline uint32_t fdiv(const FastDiv &f, uint32_t n) {
  const uint32_t t = __umulhi(f.m, n);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

// One interleave pair of [IPRM §计算原理与公式] (reading: x_rotate = (-x[2i+1], x[2i]) per pair):
//   y0 = x0*c0 + (-x1)*s0,  y1 = x1*c1 + x0*s1.
__device__ inline void rotate_pair(float a, float b, float c0, float c1, float s0, float s1,
                                   float &y0, float &y1) {
  y0 = a * c0 - b * s0;
  y1 = b * c1 + a * s1;
}

// ============================================================================================
// K1: in-place partial interleave ([IPRM §计算原理与公式], [IPRM §partial_slice 局部旋转机制]).
// A lane owns K chunks of V slice elements (V/2 pairs); chunks of one row are adjacent lanes,
// so a wavefront reads and writes whole 16-byte-aligned runs of each row's slice.  Elements
// outside [start, end) are never touched.  cos/sin rows are addressed with zero strides on
// broadcast dims (BSND, BS1D, B1ND, B11D, 111D and mixed forms).
// ============================================================================================
template <typename XT, typename CT, bool VEC>
__global__ __launch_bounds__(kBlock) void inplace_interleave_kernel(InplacePlan p) {
  constexpr int V = VEC ? Io<XT>::kPer16 : 2;
  constexpr int K = kItemsPerLane;
  const uint64_t items = uint64_t(p.items);
  const uint64_t per_block = uint64_t(kBlock) * K;
  for (uint64_t base = uint64_t(blockIdx.x) * per_block; base < items;
       base += uint64_t(gridDim.x) * per_block) {
    float xv[K][V], cv[K][V], sv[K][V];
    int64_t xoff[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint64_t it = base + uint64_t(k) * kBlock + threadIdx.x;
      xoff[k] = -1;
      if (it >= items) continue;
      uint64_t row, chunk, n, s, b;
      if (p.idx32) {
        const uint32_t i32 = uint32_t(it);
        const uint32_t r32 = fdiv(p.div_cpr, i32);
        chunk = i32 - r32 * p.chunks_per_row;
        const uint32_t bs = fdiv(p.div_n, r32);
        n = r32 - bs * uint32_t(p.N);
        const uint32_t b32 = fdiv(p.div_s, bs);
        s = bs - b32 * uint32_t(p.S);
        b = b32;
        row = r32;
      } else {
        row = it / p.chunks_per_row;
        chunk = it - row * p.chunks_per_row;
        const uint64_t bs = row / uint64_t(p.N);
        n = row - bs * uint64_t(p.N);
        b = bs / uint64_t(p.S);
        s = bs - b * uint64_t(p.S);
      }
      const int64_t crow = int64_t(b) * p.cb + int64_t(s) * p.cs + int64_t(n) * p.cn;
      const int64_t coff = crow * p.L + int64_t(chunk) * V;
      xoff[k] = int64_t(row) * p.D + p.start + int64_t(chunk) * V;
      load_n<XT, V, VEC>(p.x, xoff[k], xv[k]);
      load_n<CT, V, VEC>(p.cos, coff, cv[k]);
      load_n<CT, V, VEC>(p.sin, coff, sv[k]);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (xoff[k] < 0) continue;
      float y[V];
#pragma unroll
      for (int e = 0; e < V; e += 2)
        rotate_pair(xv[k][e], xv[k][e + 1], cv[k][e], cv[k][e + 1], sv[k][e], sv[k][e + 1], y[e],
                    y[e + 1]);
      store_n<XT, V, VEC>(p.x, xoff[k], y);
    }
  }
}

// ============================================================================================
// K2: RoPE with a cos/sin cache ([RSCC §设计动机], rope and mrope modes, NeoX and GPT-J).
// A workgroup owns a tile of tokens.  Stage: its lanes gather each token's cos|sin row from
// the cache (mrope: element i from the position row whose section holds i), raise it to
// float32 and keep it in LDS, so it is read from HBM once per token and reused by every q/k
// head.  Then lanes walk (token, head, unit) items; a unit is two V-element vectors of one
// head: rotated units take vector u and vector u + rd/(2V) of the rotated part (NeoX pairs
// lie across the two halves; GPT-J pairs lie inside each vector), pass units copy the same
// two-vector shape of [rd, H) as raw bits.  Lanes u = 0..units-1 of one head touch the head
// as two contiguous runs, so each wavefront load/store covers whole 128-byte lines.
// ============================================================================================
template <typename T, bool NEOX, bool VEC>
__global__ __launch_bounds__(kBlock) void cos_sin_cache_kernel(CachePlan p) {
  extern __shared__ float cs_tile[];  // [tile_tokens][rd]: cos (rd/2) then sin (rd/2)
  constexpr int V = Io<T>::kPer16;
  constexpr int K = kItemsPerLane;
  const int64_t rd = p.rd, half = rd / 2;
  const int64_t pass_half = (p.H - rd) / 2;
  const uint32_t ipt = p.items_per_token;
  for (int64_t tile = blockIdx.x; tile < p.tiles; tile += gridDim.x) {
    const int64_t t0 = tile * int64_t(p.tile_tokens);
    const int64_t ntok = (p.T - t0) < int64_t(p.tile_tokens) ? (p.T - t0) : int64_t(p.tile_tokens);
    const uint32_t tile_items = uint32_t(ntok) * ipt;

    // ---- stage the tile's cos|sin rows in LDS (steps 1-2: gather, split, stitch) ----
    for (int64_t idx = threadIdx.x; idx < ntok * half; idx += kBlock) {
      const int64_t tl = idx / half;
      const int64_t i = idx - tl * half;
      int sec = 0;
      if (p.mrope) {
        sec = int(i >= p.sec_end[0]) + int(i >= p.sec_end[1]);
        if (p.nsec == 4) sec += int(i >= p.sec_end[2]);
      }
      int64_t pos = p.positions[sec * p.pos_stride_row + (t0 + tl) * p.pos_stride_tok];
      pos = pos < 0 ? 0 : (pos >= p.max_seq ? p.max_seq - 1 : pos);  // never read outside
      const int64_t row = pos * p.cache_stride;
      cs_tile[tl * rd + i] = Io<T>::load1(p.cache, row + i);
      cs_tile[tl * rd + half + i] = Io<T>::load1(p.cache, row + half + i);
    }
    __syncthreads();

    // ---- step 3: rotate the first rd of every q head then k head, copy the rest ----
    for (uint32_t pbase = 0; pbase < tile_items; pbase += uint32_t(kBlock) * K) {
      RawN<T, V, VEC> va[K], vb[K];
      int64_t out_row[K], off_a[K], off_b[K];
      int32_t unit[K], tlk[K];
      bool isq[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const uint32_t it = pbase + uint32_t(k) * kBlock + threadIdx.x;
        unit[k] = -1;
        if (it >= tile_items) continue;
        const uint32_t tl = fdiv(p.div_ipt, it);
        const uint32_t r = it - tl * ipt;
        const uint32_t h = fdiv(p.div_units, r);
        const uint32_t u = r - h * p.units;
        const int64_t t = t0 + tl;
        const bool is_q = h < uint32_t(p.nq);
        const int64_t hh = is_q ? int64_t(h) : int64_t(h) - p.nq;
        const void *in = is_q ? p.q_in : p.k_in;
        const int64_t in_row = t * (is_q ? p.q_stride : p.k_stride) + hh * p.H;
        out_row[k] = t * ((is_q ? p.nq : p.nk) * p.H) + hh * p.H;
        if (u < p.rot_units) {
          off_a[k] = int64_t(u) * V;
          off_b[k] = half + int64_t(u) * V;
        } else {
          const int64_t w = int64_t(u - p.rot_units) * V;
          off_a[k] = rd + w;
          off_b[k] = rd + pass_half + w;
        }
        unit[k] = int32_t(u);
        tlk[k] = int32_t(tl);
        isq[k] = is_q;
        load_raw<T, V, VEC>(in, in_row + off_a[k], va[k]);
        load_raw<T, V, VEC>(in, in_row + off_b[k], vb[k]);
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (unit[k] < 0) continue;
        void *out = isq[k] ? p.q_out : p.k_out;
        const int64_t orow = out_row[k];
        if (uint32_t(unit[k]) >= p.rot_units) {  // pass-through: raw bits
          store_raw<T, V, VEC>(out, orow + off_a[k], va[k]);
          store_raw<T, V, VEC>(out, orow + off_b[k], vb[k]);
          continue;
        }
        float a[V], b[V], ya[V], yb[V];
        raw_to_float<T, V, VEC>(va[k], a);
        raw_to_float<T, V, VEC>(vb[k], b);
        const float *cs = cs_tile + int64_t(tlk[k]) * rd;
        if constexpr (NEOX) {
          // [RSCC §rotate_half（GPT-NeoX style）旋转模式]: x1 = a (first half), x2 = b
          const int64_t ci = int64_t(unit[k]) * V;
#pragma unroll
          for (int j = 0; j < V; ++j) {
            const float c = cs[ci + j], s = cs[half + ci + j];
            ya[j] = a[j] * c - b[j] * s;
            yb[j] = b[j] * c + a[j] * s;
          }
        } else {
          // [RSCC §rotate_interleaved（GPT-J style）旋转模式]: pairs (x[2m], x[2m+1]) inside
          // each vector; vector a holds pair indices u*V/2.., vector b holds rd/4 + u*V/2..
          const int64_t ca = int64_t(unit[k]) * (V / 2), cb = half / 2 + ca;
#pragma unroll
          for (int m = 0; m < V / 2; ++m) {
            const float c = cs[ca + m], s = cs[half + ca + m];
            ya[2 * m] = a[2 * m] * c - a[2 * m + 1] * s;
            ya[2 * m + 1] = a[2 * m + 1] * c + a[2 * m] * s;
            const float c2 = cs[cb + m], s2 = cs[half + cb + m];
            yb[2 * m] = b[2 * m] * c2 - b[2 * m + 1] * s2;
            yb[2 * m + 1] = b[2 * m + 1] * c2 + b[2 * m] * s2;
          }
        }
        store_n<T, V, VEC>(out, orow + off_a[k], ya);
        store_n<T, V, VEC>(out, orow + off_b[k], yb);
      }
    }
    __syncthreads();  // the LDS tile is rewritten by the next tile
  }
}

// ---- launch helpers -------------------------------------------------------------------------

constexpr int64_t kMaxGrid = int64_t(1) << 20;

thread_local std::string g_last_error;

int launch(const void *fn, int64_t blocks, size_t lds, void *stream, void *plan) {
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  void *args[] = {plan};
  hipError_t e = hipLaunchKernel(fn, dim3(uint32_t(blocks)), dim3(kBlock), args, lds,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = std::string("kernel launch failed: ") + hipGetErrorString(e);
    return ROPE_ERR_RUNTIME;
  }
  return ROPE_OK;
}

template <typename XT, typename CT>
const void *pick_inplace(bool vec) {
  return vec ? reinterpret_cast<const void *>(&inplace_interleave_kernel<XT, CT, true>)
             : reinterpret_cast<const void *>(&inplace_interleave_kernel<XT, CT, false>);
}

template <typename T>
const void *pick_cache(bool neox, bool vec) {
  if (neox)
    return vec ? reinterpret_cast<const void *>(&cos_sin_cache_kernel<T, true, true>)
               : reinterpret_cast<const void *>(&cos_sin_cache_kernel<T, true, false>);
  return vec ? reinterpret_cast<const void *>(&cos_sin_cache_kernel<T, false, true>)
             : reinterpret_cast<const void *>(&cos_sin_cache_kernel<T, false, false>);
}

}  // namespace
}  // namespace ropeamd

using namespace ropeamd;

#define ROPE_API extern "C" __attribute__((visibility("default")))

ROPE_API int rope_partial_inplace(const rope_tensor *x, const rope_tensor *cos,
                                  const rope_tensor *sin, int64_t rotary_mode,
                                  const int64_t *partial_slice, int64_t partial_slice_len,
                                  void *stream) {
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
  const void *fn = nullptr;
  if (plan.xdt == ROPE_F32) fn = pick_inplace<float, float>(plan.vector_io);
  else if (plan.xdt == ROPE_F16)
    fn = plan.cdt == ROPE_F32 ? pick_inplace<_Float16, float>(plan.vector_io)
                              : pick_inplace<_Float16, _Float16>(plan.vector_io);
  else
    fn = plan.cdt == ROPE_F32 ? pick_inplace<__bf16, float>(plan.vector_io)
                              : pick_inplace<__bf16, __bf16>(plan.vector_io);
  const int64_t per_block = int64_t(kBlock) * kItemsPerLane;
  return launch(fn, (plan.items + per_block - 1) / per_block, 0, stream, &plan);
}

ROPE_API int rope_with_cos_sin_cache(const rope_tensor *positions, const rope_tensor *query_in,
                                     const rope_tensor *key_in, const rope_tensor *cos_sin_cache,
                                     const int64_t *mrope_section, int64_t mrope_section_len,
                                     int64_t head_size, int is_neox_style,
                                     const rope_tensor *query_out, const rope_tensor *key_out,
                                     void *stream) {
  CachePlan plan;
  std::string err;
  const int st = plan_cache(positions, query_in, key_in, cos_sin_cache, mrope_section,
                            mrope_section_len, head_size, is_neox_style, query_out, key_out,
                            &plan, &err);
  if (st != ROPE_OK) {
    g_last_error = err;
    return st;
  }
  g_last_error.clear();
  const void *fn = plan.dt == ROPE_F32   ? pick_cache<float>(plan.neox, plan.vector_io)
                   : plan.dt == ROPE_F16 ? pick_cache<_Float16>(plan.neox, plan.vector_io)
                                         : pick_cache<__bf16>(plan.neox, plan.vector_io);
  const size_t lds = size_t(plan.tile_tokens) * size_t(plan.rd) * sizeof(float);
  return launch(fn, plan.tiles, lds, stream, &plan);
}

ROPE_API const char *rope_last_error(void) { return g_last_error.c_str(); }
