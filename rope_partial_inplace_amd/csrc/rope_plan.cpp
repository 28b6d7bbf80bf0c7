// rope_plan.cpp -- argument validation and launch planning of librope_amd.so (host only; no
// HIP call is made here, so every error path runs on a machine without a GPU).
//
// Pages:
//   [IPRM] "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码
//           接口详解与实现剖析"
//   [RSCC] "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的
//           计算原理与 aclnn 两段式调用实战"
#include <algorithm>
#include <cstdint>
#include <string>

#include "rope_plan.h"

namespace ropeamd {
namespace {

int bytes_of(rope_dtype dt) {
  switch (dt) {
    case ROPE_F32: return 4;
    case ROPE_F16: return 2;
    case ROPE_BF16: return 2;
    case ROPE_I64: return 8;
  }
  return 0;
}

bool is_float(rope_dtype dt) { return dt == ROPE_F32 || dt == ROPE_F16 || dt == ROPE_BF16; }

bool valid_rank(const rope_tensor *t) {
  if (t->ndim < 1 || t->ndim > 4) return false;
  for (int d = 0; d < t->ndim; ++d)
    if (t->shape[d] < 0) return false;
  return true;
}

// Elements of t (saturating at INT64_MAX instead of overflowing).
int64_t count(const rope_tensor *t) {
  int64_t n = 1;
  for (int d = 0; d < t->ndim; ++d)
    if (__builtin_mul_overflow(n, t->shape[d], &n)) return INT64_MAX;
  return n;
}

// The element count and the offset of the furthest element are at most 2^53 (byte offsets of
// elements of up to 8 bytes stay below 2^56, far beyond any device memory), computed without
// overflow.  A descriptor outside that cannot describe real memory, and the planning
// arithmetic on it would overflow.
bool addressable(const rope_tensor *t) {
  constexpr int64_t kLimit = int64_t(1) << 53;
  int64_t n = 1, far = 0;
  for (int d = 0; d < t->ndim; ++d) {
    int64_t off;
    if (__builtin_mul_overflow(n, t->shape[d], &n) || n > kLimit) return false;
    if (t->shape[d] == 0) continue;
    if (__builtin_mul_overflow(t->shape[d] - 1, t->stride[d], &off) || off < -kLimit ||
        off > kLimit)
      return false;
    far += off < 0 ? -off : off;  // at most 4 * 2^53: no overflow
    if (far >= kLimit) return false;
  }
  return true;
}

// Row-major contiguity; a dimension of size 1 may have any stride, and a view with no
// elements has no layout to check (reading R12: an empty x is a successful no-op).
bool row_major(const rope_tensor *t) {
  if (count(t) == 0) return true;
  int64_t want = 1;
  for (int d = t->ndim - 1; d >= 0; --d) {
    if (t->shape[d] > 1 && t->stride[d] != want) return false;
    want *= t->shape[d];
  }
  return true;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int reject(std::string *err, int code, const char *why) {
  if (err) *err = why;
  return code;
}

// Bytes [first, last) an N-d view reaches (non-negative strides).
void extent(const rope_tensor *t, uintptr_t *first, uintptr_t *last) {
  int64_t far = 0;
  for (int d = 0; d < t->ndim; ++d) far += (t->shape[d] - 1) * t->stride[d];
  *first = reinterpret_cast<uintptr_t>(t->data);
  *last = *first + uintptr_t((far + 1) * bytes_of(t->dtype));
}

bool overlap(const rope_tensor *a, const rope_tensor *b) {
  uintptr_t a0, a1, b0, b1;
  extent(a, &a0, &a1);
  extent(b, &b0, &b1);
  return a0 < b1 && b0 < a1;
}

bool identical_view(const rope_tensor *a, const rope_tensor *b) {
  if (a->data != b->data || a->ndim != b->ndim || a->dtype != b->dtype) return false;
  for (int d = 0; d < a->ndim; ++d) {
    if (a->shape[d] != b->shape[d]) return false;
    if (a->shape[d] > 1 && a->stride[d] != b->stride[d]) return false;
  }
  return true;
}

const int64_t kMropeLists[5][4] = {
    {16, 24, 24, 0}, {8, 12, 12, 0}, {24, 20, 20, 0}, {11, 11, 10, 0}, {16, 16, 16, 16}};
const int kMropeListLen[5] = {3, 3, 3, 3, 4};

}  // namespace

// Validation order: null arguments (161001) first, then dtype, mode, rank/shape, slice and
// layout checks (161002), [IPRM §返回值与错误码] and [IPRM §约束说明].
int plan_inplace(const rope_tensor *x, const rope_tensor *cos, const rope_tensor *sin,
                 int64_t rotary_mode, const int64_t *partial_slice, int64_t partial_slice_len,
                 InplacePlan *plan, std::string *err) {
  *plan = InplacePlan();
  if (x == nullptr || cos == nullptr || sin == nullptr)
    return reject(err, ROPE_ERR_PARAM_NULLPTR, "xRef, cos or sin is NULL");
  if (partial_slice == nullptr && partial_slice_len > 0)
    return reject(err, ROPE_ERR_PARAM_NULLPTR, "partial_slice is NULL with a non-zero length");
  for (const rope_tensor *t : {x, cos, sin})
    if (valid_rank(t) && count(t) > 0 && t->data == nullptr)
      return reject(err, ROPE_ERR_PARAM_NULLPTR, "a non-empty tensor has NULL data");

  if (!is_float(x->dtype)) return reject(err, ROPE_ERR_PARAM_INVALID, "xRef dtype unsupported");
  if (cos->dtype != sin->dtype)
    return reject(err, ROPE_ERR_PARAM_INVALID, "cos and sin dtypes differ");
  if (cos->dtype != x->dtype && cos->dtype != ROPE_F32)
    return reject(err, ROPE_ERR_PARAM_INVALID, "cos/sin must have xRef's dtype or float32");
  // rotary_mode ([IPRM §参数说明]): 1 interleave; 0 half mode, which the pages list but
  // have not enabled -- enabled here with x1, x2 the two halves of the slice.
  if (rotary_mode != 0 && rotary_mode != 1)
    return reject(err, ROPE_ERR_PARAM_INVALID, "rotary_mode must be 1 (interleave) or 0 (half)");

  for (const rope_tensor *t : {x, cos, sin})
    if (!valid_rank(t) || t->ndim != 4)
      return reject(err, ROPE_ERR_PARAM_INVALID, "xRef, cos and sin must be 4-D");
  for (const rope_tensor *t : {x, cos, sin})
    if (!addressable(t))
      return reject(err, ROPE_ERR_PARAM_INVALID, "tensor extent beyond 2^56 elements or bytes");
  for (int d = 0; d < 4; ++d)
    if (cos->shape[d] != sin->shape[d])
      return reject(err, ROPE_ERR_PARAM_INVALID, "cos and sin shapes differ");
  const int64_t D = x->shape[3];
  if (D > 1024) return reject(err, ROPE_ERR_PARAM_INVALID, "D > 1024");
  if (D % 2 != 0) return reject(err, ROPE_ERR_PARAM_INVALID, "D is odd");

  int64_t start = 0, end = D;
  if (partial_slice != nullptr || partial_slice_len != 0) {
    if (partial_slice_len != 2)
      return reject(err, ROPE_ERR_PARAM_INVALID, "partial_slice must hold 2 values");
    start = partial_slice[0];
    end = partial_slice[1];
  }
  if (start < 0 || end < 0 || end > D || end < start)
    return reject(err, ROPE_ERR_PARAM_INVALID, "partial_slice out of range");
  const int64_t L = end - start;
  if (L % 2 != 0) return reject(err, ROPE_ERR_PARAM_INVALID, "slice length is odd");
  if (!row_major(x) || !row_major(cos) || !row_major(sin))
    return reject(err, ROPE_ERR_PARAM_INVALID, "non-contiguous tensors are not supported");

  if (L == 0) {  // empty slice: no-op, before the cos/sin last-dim check
    plan->noop = true;
    return ROPE_OK;
  }
  if (cos->shape[3] != L)
    return reject(err, ROPE_ERR_PARAM_INVALID, "cos/sin last dim != slice length");
  for (int d = 0; d < 3; ++d)
    if (cos->shape[d] != 1 && cos->shape[d] != x->shape[d])
      return reject(err, ROPE_ERR_PARAM_INVALID, "cos/sin do not broadcast to xRef");

  InplacePlan &p = *plan;
  p.half = rotary_mode == 0;
  p.xdt = x->dtype;
  p.cdt = cos->dtype;
  p.x = x->data;
  p.cos = cos->data;
  p.sin = sin->data;
  p.B = x->shape[0];
  p.S = x->shape[1];
  p.N = x->shape[2];
  p.D = D;
  p.start = start;
  p.L = L;
  p.rows = p.B * p.S * p.N;
  if (p.rows == 0) {
    p.noop = true;
    return ROPE_OK;
  }
  // x is written in place while other lanes read cos/sin: no shared memory (cos and sin are
  // only read and may share memory with each other).
  if (overlap(x, cos) || overlap(x, sin))
    return reject(err, ROPE_ERR_PARAM_INVALID, "xRef overlaps cos or sin");
  const int64_t Sc = cos->shape[1], Nc = cos->shape[2];
  p.cn = cos->shape[2] == 1 ? 0 : 1;
  p.cs = cos->shape[1] == 1 ? 0 : Nc;
  p.cb = cos->shape[0] == 1 ? 0 : Sc * Nc;
  const bool bs_stream = (cos->shape[0] == p.B || p.B == 1) && (cos->shape[1] == p.S || p.S == 1);

  // Lane chunks of V elements: a 16-byte access for the wider of x and cos/sin (8 bytes for
  // the narrower) when every chunk start is aligned to its access size; else element access.
  // Half mode: a lane owns chunk u of each half (its pairs are (i, i + L/2)), so the halves
  // must split into whole chunks.
  const int xs = bytes_of(p.xdt), cs = bytes_of(p.cdt);
  const int64_t v = 16 / std::max(xs, cs);
  const int64_t span = p.half ? L / 2 : L;  // elements one lane's chunks are taken from
  const bool aligned = span % v == 0 && (D * xs) % (v * xs) == 0 &&
                       (start * xs) % (v * xs) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.x) % uintptr_t(v * xs)) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.cos) % uintptr_t(v * cs)) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.sin) % uintptr_t(v * cs)) == 0;
  p.vector_io = aligned;
  p.vec = aligned ? uint32_t(v) : (p.half ? 1u : 2u);
  p.chunks_per_row = uint32_t(span / p.vec);
  // Half mode, vector path, 1..16 chunks per half: one chunk per lane, the pair partner in
  // lane (lane ^ P) with P the chunk count of a half rounded up to a power of two; the lanes
  // of a row past a half's last chunk carry none.  Each access then covers a row's slice as
  // one contiguous run, where a lane owning a chunk of both halves covered each half apart:
  // bf16 x [4,4096,32,96] (12 chunks per half) measured 44.4 us that way.
  const uint32_t cph = p.chunks_per_row;
  uint32_t pw = 1;
  while (pw < cph) pw <<= 1;
  if (p.half && aligned && cph >= 1 && pw <= 16) {
    p.xch = pw;
    p.xch_cph = cph;
    p.chunks_per_row = 2 * pw;
  }
  // Heads per lane: with cos/sin broadcast over N, a lane rotates its chunk in nhl consecutive
  // heads with one cos/sin load: the larger of 4, 2 that divides N and keeps a lane's x
  // bytes at 32 or less (measured best: 4 heads of 8-byte chunks, 2 of 16-byte ones; more
  // heads per lane leave too few lanes).  Vector path only.
  p.nhl = 1;
  const uint32_t x_bytes_per_head = p.vec * uint32_t(xs) * (p.half && p.xch == 0 ? 2u : 1u);
  if (p.cn == 0 && p.N > 1 && p.vector_io)
    for (uint32_t c : {4u, 2u})
      if (p.N % c == 0 && c * x_bytes_per_head <= 32) {
        p.nhl = c;
        break;
      }
  // cos/sin are streamed (non-temporal) when each cos/sin row is read by one lane group only
  p.cos_stream = bs_stream && (cos->shape[2] == p.N || p.N == int64_t(p.nhl));
  const int64_t ng = p.N / p.nhl;
  p.items = p.B * p.S * ng * p.chunks_per_row;
  // 32-bit item indices: an index below 2^31 plus the grid stride (at most kMaxGrid * kBlock
  // = 2^30 lanes) stays below 2^32, so a lane's index never wraps round to a low item.
  p.idx32 = p.items <= (int64_t(1) << 31);
  uint32_t block = kBlock;
  while (block > uint32_t(kBlockMin) && p.items < kComputeUnits * int64_t(block)) block /= 2;
  p.block = p.items > kOneRoundLanes ? uint32_t(kBlockMulti) : block;
  p.div_cpr = make_fastdiv(p.chunks_per_row);
  p.div_ng = make_fastdiv(uint32_t(std::min<int64_t>(ng, 0xffffffff)));
  if (ng > 0xffffffffLL || p.S > 0xffffffffLL || int64_t(p.nhl) * D > 0xffffffffLL)
    p.idx32 = false;
  if (p.idx32) {
    // cos/sin row = r*a + (r / ng)*bq + (r / (ng*S))*c (InplacePlan::crow_a); ng * S is at most
    // the item count, so both divisors fit 32 bits.  Terms that coincide are merged: with
    // B = 1, b = r / (ng*S) is 0; with S = 1, r / (ng*S) = r / ng; with ng = 1, r / ng = r.
    int64_t a = int64_t(p.nhl) * p.cn;
    int64_t bq = p.cs - ng * a;
    int64_t c = p.cb - p.S * p.cs;
    if (p.B == 1) c = 0;
    if (p.S == 1) {
      bq += c;
      c = 0;
    }
    if (ng == 1) {
      a += bq;
      bq = 0;
    }
    p.crow_a = uint32_t(a);
    p.crow_b = uint32_t(bq);
    p.crow_c = uint32_t(c);
    p.div_ngs = make_fastdiv(uint32_t(ng * p.S));
  }
  return ROPE_OK;
}

// [RSCC §入参校验逻辑] (null, dtype, shape, mropeSection checks) and [RSCC §约束说明]
// (64-byte alignment of headSize and rotaryDim, rotaryDim <= headSize).
int plan_cache(const rope_tensor *positions, const rope_tensor *query_in,
               const rope_tensor *key_in, const rope_tensor *cache,
               const int64_t *mrope_section, int64_t mrope_section_len, int64_t head_size,
               int is_neox_style, int64_t cache_mode, const rope_tensor *query_out,
               const rope_tensor *key_out, CachePlan *plan, std::string *err) {
  *plan = CachePlan();
  const rope_tensor *all[6] = {positions, query_in, key_in, cache, query_out, key_out};
  for (const rope_tensor *t : all)
    if (t == nullptr) return reject(err, ROPE_ERR_PARAM_NULLPTR, "a tensor argument is NULL");
  if (mrope_section == nullptr && mrope_section_len > 0)
    return reject(err, ROPE_ERR_PARAM_NULLPTR, "mrope_section is NULL with a non-zero length");
  if (mrope_section_len < 0)
    return reject(err, ROPE_ERR_PARAM_INVALID, "negative mrope_section length");
  for (const rope_tensor *t : all)
    if (valid_rank(t) && count(t) > 0 && t->data == nullptr)
      return reject(err, ROPE_ERR_PARAM_NULLPTR, "a non-empty tensor has NULL data");

  if (positions->dtype != ROPE_I64)
    return reject(err, ROPE_ERR_PARAM_INVALID, "positions must be int64");
  const rope_dtype dt = query_in->dtype;
  if (!is_float(dt)) return reject(err, ROPE_ERR_PARAM_INVALID, "queryIn dtype unsupported");
  for (const rope_tensor *t : {key_in, cache, query_out, key_out})
    if (t->dtype != dt)
      return reject(err, ROPE_ERR_PARAM_INVALID, "all float tensors must share queryIn's dtype");

  for (const rope_tensor *t : {query_in, key_in, cache, query_out, key_out})
    if (!valid_rank(t) || t->ndim != 2)
      return reject(err, ROPE_ERR_PARAM_INVALID, "queryIn, keyIn, cache and outputs must be 2-D");
  if (!valid_rank(positions)) return reject(err, ROPE_ERR_PARAM_INVALID, "bad positions shape");
  for (const rope_tensor *t : all)
    if (!addressable(t))
      return reject(err, ROPE_ERR_PARAM_INVALID, "tensor extent beyond 2^56 elements or bytes");
  for (const rope_tensor *t : {query_in, key_in, cache})
    if (t->shape[0] == 0 || t->shape[1] == 0)
      return reject(err, ROPE_ERR_PARAM_INVALID, "queryIn, keyIn and cache must be non-empty");
  if (key_in->shape[0] != query_in->shape[0])
    return reject(err, ROPE_ERR_PARAM_INVALID, "keyIn and queryIn differ in token count");
  for (int d = 0; d < 2; ++d)
    if (query_out->shape[d] != query_in->shape[d] || key_out->shape[d] != key_in->shape[d])
      return reject(err, ROPE_ERR_PARAM_INVALID, "output shape differs from input shape");

  const int64_t T = query_in->shape[0];
  const int64_t rd = cache->shape[1];

  bool mrope = false;
  int nsec = 0;
  int64_t sec[4] = {0, 0, 0, 0};
  if (mrope_section_len > 0) {
    if (mrope_section_len != 3 && mrope_section_len != 4)
      return reject(err, ROPE_ERR_PARAM_INVALID, "mrope_section needs 3 or 4 entries");
    int64_t total = 0;
    for (int64_t i = 0; i < mrope_section_len; ++i) {
      if (mrope_section[i] < 0 || mrope_section[i] > rd)
        return reject(err, ROPE_ERR_PARAM_INVALID, "mrope_section entry outside [0, rotaryDim]");
      total += mrope_section[i];
    }
    if (mrope_section[0] > 0) {
      if (2 * total != rd)
        return reject(err, ROPE_ERR_PARAM_INVALID, "2*sum(mrope_section) != rotaryDim");
      bool found = false;
      for (int w = 0; w < 5 && !found; ++w) {
        if (kMropeListLen[w] != mrope_section_len) continue;
        found = std::equal(mrope_section, mrope_section + mrope_section_len, kMropeLists[w]);
      }
      if (!found)
        return reject(err, ROPE_ERR_PARAM_INVALID, "mrope_section is not a supported list");
      mrope = true;
      nsec = int(mrope_section_len);
      for (int i = 0; i < nsec; ++i) sec[i] = mrope_section[i];
    }
  }

  // cacheMode ([RSCC §V2 接口：cacheMode 扩展]): 0 sectioned, 1 interleaved; the 4-section
  // list allows 0 only; in rope mode the value has no effect.
  if (cache_mode != 0 && cache_mode != 1)
    return reject(err, ROPE_ERR_PARAM_INVALID, "cacheMode must be 0 or 1");
  if (mrope && cache_mode == 1 && nsec == 4)
    return reject(err, ROPE_ERR_PARAM_INVALID, "cacheMode 1 needs a 3-section mropeSection");

  const int es = bytes_of(dt);
  const int64_t align_elems = 64 / es;
  if (head_size <= 0 || head_size % align_elems != 0)
    return reject(err, ROPE_ERR_PARAM_INVALID, "headSize must be a positive 64-byte multiple");
  if (query_in->shape[1] % head_size != 0 || key_in->shape[1] % head_size != 0)
    return reject(err, ROPE_ERR_PARAM_INVALID, "q/k widths are not multiples of headSize");
  if (rd > head_size || rd % align_elems != 0)
    return reject(err, ROPE_ERR_PARAM_INVALID, "rotaryDim must be a 64-byte multiple <= headSize");

  if (!mrope) {
    if (positions->ndim != 1 || positions->shape[0] != T)
      return reject(err, ROPE_ERR_PARAM_INVALID, "rope mode: positions must be [numTokens]");
  } else if (positions->ndim != 2 || positions->shape[0] != nsec || positions->shape[1] != T) {
    return reject(err, ROPE_ERR_PARAM_INVALID, "mrope mode: positions must be [m, numTokens]");
  }

  for (const rope_tensor *t : {query_in, key_in, cache})
    if (t->stride[1] != 1 || t->stride[0] < 0)
      return reject(err, ROPE_ERR_PARAM_INVALID, "inputs need unit inner and non-negative row stride");
  for (int d = 0; d < positions->ndim; ++d)
    if (positions->stride[d] < 0)
      return reject(err, ROPE_ERR_PARAM_INVALID, "negative positions stride");
  if (!row_major(query_out) || !row_major(key_out))
    return reject(err, ROPE_ERR_PARAM_INVALID, "queryOut/keyOut must be contiguous");

  if (overlap(query_out, key_out))
    return reject(err, ROPE_ERR_PARAM_INVALID, "queryOut and keyOut overlap");
  const rope_tensor *inputs[4] = {positions, query_in, key_in, cache};
  const rope_tensor *outputs[2] = {query_out, key_out};
  for (int o = 0; o < 2; ++o)
    for (int i = 0; i < 4; ++i) {
      if (!overlap(outputs[o], inputs[i])) continue;
      const bool own_input = (o == 0 && i == 1) || (o == 1 && i == 2);
      if (own_input && identical_view(outputs[o], inputs[i])) continue;
      return reject(err, ROPE_ERR_PARAM_INVALID, "an output overlaps another tensor");
    }

  CachePlan &p = *plan;
  p.dt = dt;
  p.neox = is_neox_style != 0;
  p.mrope = mrope;
  p.positions = static_cast<const int64_t *>(positions->data);
  p.q_in = query_in->data;
  p.k_in = key_in->data;
  p.cache = cache->data;
  p.q_out = query_out->data;
  p.k_out = key_out->data;
  p.T = T;
  p.H = head_size;
  p.rd = rd;
  p.nq = query_in->shape[1] / head_size;
  p.nk = key_in->shape[1] / head_size;
  p.max_seq = cache->shape[0];
  p.q_stride = query_in->stride[0];
  p.k_stride = key_in->stride[0];
  p.cache_stride = cache->stride[0];
  if (mrope) {
    p.pos_stride_row = positions->stride[0];
    p.pos_stride_tok = positions->stride[1];
  } else {
    p.pos_stride_row = 0;
    p.pos_stride_tok = positions->stride[0];
  }
  p.nsec = nsec;
  int64_t acc = 0;
  for (int i = 0; i < nsec; ++i) {
    acc += sec[i];
    p.sec_end[i] = int32_t(acc);
  }

  // 16-byte vectors when every row start and base pointer is 16-byte aligned.
  const bool ok16 = aligned16(p.q_in) && aligned16(p.k_in) && aligned16(p.q_out) &&
                    aligned16(p.k_out) && (p.q_stride * es) % 16 == 0 &&
                    (p.k_stride * es) % 16 == 0;
  p.vector_io = ok16;
  p.vec = uint32_t(16 / es);  // headSize and rotaryDim are 64-byte multiples: always divides
  // NeoX pairs lie rd/2 apart, so a NeoX unit is two vectors (u and u + rd/(2 vec)); GPT-J
  // pairs lie inside one vector, so a GPT-J unit is one vector and a head's units run
  // contiguously.  Each access instruction then covers whole lines of the head.
  const int64_t per_unit = p.neox ? 2 * p.vec : p.vec;
  p.units = uint32_t(head_size / per_unit);
  p.rot_units = uint32_t(rd / per_unit);
  const int64_t ipt = (p.nq + p.nk) * int64_t(p.units);
  if (ipt > 0x7fffffffLL)
    return reject(err, ROPE_ERR_PARAM_INVALID, "too many heads per token for this library");
  p.items_per_token = uint32_t(ipt);
  // Tokens per workgroup: the tile's items are processed in passes of kBlock*K; pick the
  // smallest tile that fills its passes to >= 90% (at most 8 passes), else the best filled
  // one.  The LDS tile holds tile_tokens * rd elements of the cache type; it is sized here
  // as if they were 4-byte floats (an upper bound), within 32 KiB.
  const int64_t pass = int64_t(kCacheBlock) * (p.neox ? kNeoxItemsPerLane : kGptjItemsPerLane);
  const int64_t tt_lds = std::max<int64_t>(1, (32 * 1024) / (rd * 4));
  int64_t tt = 1;
  double best = -1.0;
  for (int64_t cand = 1; cand <= std::min<int64_t>(tt_lds, 64); ++cand) {
    const int64_t items = cand * ipt;
    const int64_t passes = (items + pass - 1) / pass;
    if (passes > 8 && cand > 1) break;
    const double fill = double(items) / double(passes * pass);
    if (fill > best + 1e-9) {
      best = fill;
      tt = cand;
    }
    if (fill >= 0.9) break;
  }
  tt = std::min<int64_t>(tt, T);
  if (T <= kOneRoundCacheTiles) tt = 1;
  // A token's cos|sin row of more than 16384 elements does not fit the 64 KiB LDS tile: such
  // plans stage nothing and read each item's cos/sin from the cache row directly.  Only rope
  // mode gets there (every mrope list has rotaryDim = 2 * sum <= 128).
  p.cs_direct = rd * 4 * tt > 64 * 1024;
  if (p.cs_direct && mrope)
    return reject(err, ROPE_ERR_PARAM_INVALID, "internal: mrope plan with a direct cos/sin read");
  p.tile_tokens = uint32_t(tt);
  p.tiles = (T + tt - 1) / tt;
  // Tapered end: a workgroup lives for a few loaded round trips, and the last round drains
  // at falling occupancy; one-token tiles for the last ~round of tokens shorten that drain.
  p.big_tiles = p.tiles;
  p.big_tokens = T;
  if (tt > 1) {
    const int64_t taper = std::min<int64_t>(kTaperTokens, T / 4);
    p.big_tiles = (T - taper) / tt;
    p.big_tokens = p.big_tiles * tt;
    p.tiles = p.big_tiles + (T - p.big_tokens);
  }
  p.div_units = make_fastdiv(p.units);
  p.div_ipt = make_fastdiv(p.items_per_token);
  p.cache_vec = aligned16(p.cache) && (p.cache_stride * es) % 16 == 0;
  p.stage_chunks = uint32_t((rd / 2) / p.vec);  // rd/2 is a 32-byte multiple
  p.div_stage = make_fastdiv(p.stage_chunks);
  // Interleaved stitching: element i of cos/sin takes row 1 if i % 3 == 1 and row 2 if
  // i % 3 == 2, below 3 * mropeSection[1] (the bound printed for both rows; for every accepted
  // list it selects the same elements as 3 * mropeSection[2], the slices ending at rd/2).
  p.interleaved = mrope && cache_mode == 1;
  p.interleave_end = p.interleaved ? int32_t(3 * sec[1]) : 0;
  bool split = false;
  for (int i = 0; i + 1 < nsec; ++i) split |= (p.sec_end[i] % int32_t(p.vec)) != 0;
  p.multi_row = p.interleaved || (mrope && split);
  // The multi-row staging reads rows 0..2; only the 3-section lists get there (the 4-section
  // list has its boundaries on vector edges and allows cacheMode 0 only).
  if (p.multi_row && nsec != 3)
    return reject(err, ROPE_ERR_PARAM_INVALID, "mropeSection layout not supported");
  // The wavefront path needs 16-byte q/k and cache access, a head of at most 64 units (one
  // row of lanes), positions readable as aligned 8-byte words (they go through the scalar
  // cache), and a wave count that fits its 32-bit index.
  // NeoX layouts.  Each access instruction should cover whole 128-byte lines of the heads:
  //  - pair units (two vectors, i and i + rd/2, per lane) span rd/2 elements of a head per
  //    access: taken when that is a whole number of lines;
  //  - otherwise, with rd <= H/2, the exchange layout (accesses span H/2) when that is whole
  //    lines;
  //  - otherwise one-vector units (accesses span whole heads).
  // Measured with bf16 q/k: rd 64 or 32 of H 128 36.7-43.2 -> 29.8-30.0 us with the exchange
  // layout; rd 96 of H 128 43.0 -> 33.1 us and H = rd = 64 36.2 -> 31.4 us with one-vector
  // units (28.5 and 28.4 us once a pair's lanes shared the cos|sin gather).  On whole-line
  // shapes one-vector units stay 1-2% slower than pair units in rope and three-section mrope,
  // 26% with multi-row stitching.
  const int64_t line = 128;
  const bool pair_lines = (rd / 2 * es) % line == 0;
  const bool xch = p.neox && !pair_lines && 2 * rd <= head_size && (head_size / 2 * es) % line == 0;
  const bool lin = p.neox && !pair_lines && !xch && 2 * p.units <= 64;
  const uint32_t lanes = lin ? 2 * p.units : p.units;  // lanes per head
  // Its stores address one token's q or k output row as a buffer range of 32-bit offsets.
  const int64_t row_limit = int64_t(1) << 31;
  const bool rows_fit = p.nq * head_size * es < row_limit && p.nk * head_size * es < row_limit;
  if (p.vector_io && p.cache_vec && lanes >= 1 && lanes <= 64 && rows_fit &&
      (reinterpret_cast<uintptr_t>(p.positions) & 7u) == 0) {
    const uint32_t rows =
        p.neox && !xch && !lin && !p.multi_row ? kWaveRowsPairUnits : kWaveRowsVectorUnits;
    const uint32_t hpw = 64u / lanes;
    const uint32_t heads = rows * hpw;
    const int64_t wpt = (p.nq + p.nk + heads - 1) / heads;
    if (wpt <= int64_t(0x7fffffff) && T <= kMaxWaves / wpt) {
      p.wave = true;
      p.wave_rows = rows;
      p.wave_block = uint32_t(p.neox ? kWaveBlockNeox : kWaveBlockGptj);
      p.wave_hpw = hpw;
      p.wave_heads = heads;
      p.wave_wpt = uint32_t(wpt);
      p.waves = T * wpt;
      p.wave_scalar_row = !p.neox && !p.mrope && rd * es == kScalarRowBytes &&
                          p.waves >= kScalarRowMinWaves;
      p.div_wpt = make_fastdiv(p.wave_wpt);
      p.wave_lin = lin;
      p.wave_xch = xch;
    }
  }
  return ROPE_OK;
}

}  // namespace ropeamd
