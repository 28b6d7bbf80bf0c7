/*
 * rope.h -- C ABI of the MI355X (gfx950) RoPE apply library, librope_amd.so.
 *
 * Each operation is one call that validates its arguments on the host and then enqueues
 * hand-written HIP kernels on the caller's stream:
 *
 *   rope_partial_inplace           in-place partial RoPE (interleave or half mode) on a BSND tensor
 *   rope_partial_inplace_backward  its gradient with respect to x, in place on the gradient
 *   rope_with_cos_sin_cache        RoPE of query/key rows with cos/sin gathered from a cache by
 *                                  position; rope or mrope mode; GPT-NeoX or GPT-J style
 *   rope_with_cos_sin_cache_v2     the same with the cacheMode argument (sectioned or
 *                                  interleaved mrope stitching)
 *
 * Pages defining the operations:
 *   [IPRM] "CANN ops-transformer 的 aclnnInplacePartialRotaryMul 算子：Inplace 部分旋转位置编码
 *           接口详解与实现剖析"
 *   [RSCC] "CANN ops-transformer 旋转位置编码算子 RopeWithSinCosCache 深度解析：cache 化 RoPE 的
 *           计算原理与 aclnn 两段式调用实战"
 * Both pages describe a two-phase interface (workspace size, then execute).  These kernels
 * need no workspace, so the two phases are one call here.
 *
 * Common rules
 *  - Memory: every tensor `data` pointer is device memory (or memory the GPU can address)
 *    owned by the caller.  The library never allocates, frees, retains a pointer after the
 *    call returns, or synchronizes.  Host arrays (partial_slice, mrope_section) are read
 *    during the call only.
 *  - Stream: `stream` is a hipStream_t (NULL = the null stream of the current device).  The
 *    kernels run on the current HIP device: the stream and every tensor must belong to it
 *    (hipSetDevice first when several GPUs are in use).  The
 *    call returns once the work is enqueued; results are visible after the stream is
 *    synchronized.  The library is stateless and reentrant; calls that touch the same
 *    buffers must be ordered by the caller (same stream or events).
 *  - Arithmetic: operands are raised to float32, each product and each sum of the formulas
 *    is one float32 operation (no fused multiply-add), and the result is rounded once to
 *    the tensor dtype (round to nearest even).  Data outside the rotated range is never
 *    converted: it is left untouched (in-place op) or copied bit for bit (cache op).
 *  - Errors: a non-zero status means nothing was enqueued and no buffer was touched
 *    (except ROPE_ERR_RUNTIME, which reports a failed launch).  rope_last_error() gives a
 *    text for the last failing call of the calling thread.
 *  - Determinism: every output element is written by exactly one GPU lane with no atomics,
 *    so repeated calls give bit-identical results ([IPRM §约束说明], [RSCC §约束说明]).
 */
#ifndef ROPE_AMD_H
#define ROPE_AMD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of a tensor description. */
typedef enum {
  ROPE_F32 = 0,  /* IEEE binary32 */
  ROPE_F16 = 1,  /* IEEE binary16 */
  ROPE_BF16 = 2, /* bfloat16 */
  ROPE_I64 = 3   /* int64 (positions) */
} rope_dtype;

/* Status codes.  The two parameter codes are the ones of [IPRM §返回值与错误码];
 * ROPE_ERR_RUNTIME has no value on the pages (library-defined). */
enum {
  ROPE_OK = 0,
  ROPE_ERR_PARAM_NULLPTR = 161001, /* a required tensor (or its data) is NULL          */
  ROPE_ERR_PARAM_INVALID = 161002, /* dtype / shape / attribute / layout not supported */
  ROPE_ERR_RUNTIME = 361001        /* the HIP launch failed                           */
};

/* A strided tensor view.  shape[] and stride[] hold `ndim` entries (1..4); strides are in
 * elements.  `data` may be NULL only when the tensor has no elements.  Every entry point
 * refuses (ROPE_ERR_PARAM_INVALID) a view with more than 2^53 elements or whose furthest
 * element lies 2^53 or more elements from its first: no buffer is that large. */
typedef struct {
  void *data;
  rope_dtype dtype;
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} rope_tensor;

/*
 * rope_partial_inplace -- in-place partial RoPE.
 *
 * Defined in [IPRM §计算原理与公式] and [IPRM §partial_slice 局部旋转机制]: on the slice
 * x[..., start:end) of the last dim (indices below count from `start`), x = x*cos +
 * x_rotate*sin.  Interleave mode (rotary_mode 1): x_rotate = (-x2, x1) interleaved per pair,
 * so each pair (x[2i], x[2i+1]) becomes
 *     x[2i]   = x[2i]*cos[2i]     - x[2i+1]*sin[2i]
 *     x[2i+1] = x[2i+1]*cos[2i+1] + x[2i]*sin[2i+1]
 * Half mode (rotary_mode 0; [IPRM §参数说明] lists it as not yet enabled on its hardware,
 * enabled here): x1, x2 are the two halves of the slice, x_rotate = cat(-x2, x1), so with
 * h = L/2 each pair (x[i], x[i+h]) becomes
 *     x[i]   = x[i]*cos[i]     - x[i+h]*sin[i]
 *     x[i+h] = x[i+h]*cos[i+h] + x[i]*sin[i+h]
 * Elements in [0, start) and [end, D) are never read or written.
 *
 * x      [B, S, N, D] (BSND), contiguous, F32 / F16 / BF16; read and written in place.
 * cos,   [Bc, Sc, Nc, L] with L = end - start, contiguous, both of one dtype: x's dtype or
 * sin    F32 (F32 with half-precision x is the mixed case of [IPRM §返回值与错误码]).
 *        Each of Bc, Sc, Nc is 1 (broadcast) or equal to x's B, S, N; this covers the BSND,
 *        BS1D, B1ND, B11D and 111D layouts of [IPRM §约束说明].
 * rotary_mode    1 (interleave) or 0 (half); any other value is ROPE_ERR_PARAM_INVALID.
 * partial_slice  host array {start, end}; NULL with partial_slice_len 0 means [0, D).
 *                0 <= start <= end <= D and end - start even; start == end returns
 *                ROPE_OK at once without launching anything (and without checking cos/sin's
 *                last dim).  start may be odd.
 * Constraints (else ROPE_ERR_PARAM_INVALID): 4-D tensors, D even and D <= 1024, cos and
 * sin of one shape whose last dim is L, contiguous tensors, and x sharing no memory with
 * cos or sin (cos and sin may be one tensor).  NULL x/cos/sin, or NULL data
 * of a non-empty tensor, gives ROPE_ERR_PARAM_NULLPTR.  An x with no elements is a no-op.
 */
int rope_partial_inplace(const rope_tensor *x, const rope_tensor *cos, const rope_tensor *sin,
                         int64_t rotary_mode, const int64_t *partial_slice,
                         int64_t partial_slice_len, void *stream);

/*
 * rope_partial_inplace_backward -- gradient of rope_partial_inplace with respect to x, in place
 * on the incoming gradient g.
 *
 * [IPRM §Python 接口与自动微分]: the training path computes the gradient of x with a backward
 * op; cos and sin get no gradient; empty tensors and empty slices are no-ops.  The pages give
 * no formula: on each slice pair (j, k) -- (2i, 2i+1) in interleave mode, (i, i+L/2) in half
 * mode -- the forward map is y = [[c_j, -s_j], [s_k, c_k]] x, so its gradient is the transpose,
 *     g[j] = g[j]*cos[j] + g[k]*sin[k]
 *     g[k] = g[k]*cos[k] - g[j]*sin[j]
 * and elements outside [start, end) pass the gradient through unchanged (never touched).
 * Arguments, layouts, validation, error codes and the no-op rules are those of
 * rope_partial_inplace, with g in the place of x.
 */
int rope_partial_inplace_backward(const rope_tensor *g, const rope_tensor *cos,
                                  const rope_tensor *sin, int64_t rotary_mode,
                                  const int64_t *partial_slice, int64_t partial_slice_len,
                                  void *stream);

/*
 * rope_with_cos_sin_cache -- RoPE with a cos/sin cache ([RSCC §设计动机]).
 *
 * For each token t: cos/sin are gathered from cos_sin_cache[position] and split in halves
 * (first rotaryDim/2 columns cos, last rotaryDim/2 sin).  Every head of query, then of key,
 * has its first rotaryDim elements rotated and the remaining headSize - rotaryDim copied:
 *   GPT-NeoX (is_neox_style != 0, [RSCC §rotate_half（GPT-NeoX style）旋转模式]):
 *       x1 = x[0 : rd/2], x2 = x[rd/2 : rd]
 *   GPT-J    (is_neox_style == 0, [RSCC §rotate_interleaved（GPT-J style）旋转模式]):
 *       x1 = x[0 : rd : 2], x2 = x[1 : rd : 2], outputs interleaved back
 *   o1 = x1*cos - x2*sin,  o2 = x2*cos + x1*sin.
 *
 * positions      INT64. rope mode: [T]. mrope mode: [m, T] with m = mrope_section_len.
 *                Any non-negative strides.  Every value must lie in [0, maxSeqLen) -- a
 *                precondition ([RSCC §约束说明]) that is not checked (that would need a device
 *                synchronization); a value outside it is clamped into range on the device, so
 *                the call never reads outside the cache but its output is then meaningless.
 * query_in       [T, Nq*headSize], key_in [T, Nk*headSize]: F32 / F16 / BF16, unit inner
 *                stride, any non-negative row stride (the qStride/kStride of the pages).
 * cos_sin_cache  [maxSeqLen, rotaryDim], same dtype, unit inner stride, any row stride.
 * mrope_section  host array or NULL.  NULL (length 0) -> rope mode.  Otherwise 3 or 4
 *                non-negative entries; entry 0 > 0 selects mrope ([RSCC §rope 模式：标准位置编码]),
 *                where 2*sum == rotaryDim and the list is one of {16,24,24}, {8,12,12},
 *                {24,20,20}, {11,11,10}, {16,16,16,16} ([RSCC §入参校验逻辑]).  Element i of
 *                cos/sin then comes from the position row k whose section holds i
 *                ([RSCC §mrope 模式：多模态位置编码]).  Entry 0 == 0 -> rope mode.
 * head_size      headSize; a positive multiple of 64 bytes (32 elements for F16/BF16, 16 for
 *                F32); rotaryDim (= cache width) is a multiple of 64 bytes too and
 *                <= headSize ([RSCC §约束说明]).
 * query_out,     contiguous, same shapes and dtype as the inputs.  An output may be its own
 * key_out        input exactly (same pointer and layout); any other overlap between an
 *                output and another tensor is rejected.
 * Errors: NULL tensors -> ROPE_ERR_PARAM_NULLPTR; wrong dtype, rank, empty inputs, token
 * count mismatch, output shape mismatch, bad mropeSection or alignment -> ROPE_ERR_PARAM_INVALID.
 */
int rope_with_cos_sin_cache(const rope_tensor *positions, const rope_tensor *query_in,
                            const rope_tensor *key_in, const rope_tensor *cos_sin_cache,
                            const int64_t *mrope_section, int64_t mrope_section_len,
                            int64_t head_size, int is_neox_style,
                            const rope_tensor *query_out, const rope_tensor *key_out,
                            void *stream);

/*
 * rope_with_cos_sin_cache_v2 -- rope_with_cos_sin_cache with the cacheMode argument
 * ([RSCC §V2 接口：cacheMode 扩展]), which picks how mrope stitches cos/sin from the position
 * rows:
 *   cache_mode 0  sectioned: element i comes from the row whose section holds i (exactly
 *                 rope_with_cos_sin_cache, which is this call with cache_mode 0);
 *   cache_mode 1  interleaved, 3-section lists only: every element starts from row 0; then
 *                 the elements i < 3*mropeSection[1] with i % 3 == 1 come from row 1 and
 *                 those with i % 3 == 2 from row 2 (index i in [0, rotaryDim/2), the same
 *                 for the cos and the sin half).
 * cache_mode must be 0 or 1, and 0 with the list {16,16,16,16}; anything else gives
 * ROPE_ERR_PARAM_INVALID (checked in rope mode too, where the value changes nothing).
 * Every other argument, layout and rule is that of rope_with_cos_sin_cache.
 */
int rope_with_cos_sin_cache_v2(const rope_tensor *positions, const rope_tensor *query_in,
                               const rope_tensor *key_in, const rope_tensor *cos_sin_cache,
                               const int64_t *mrope_section, int64_t mrope_section_len,
                               int64_t head_size, int is_neox_style, int64_t cache_mode,
                               const rope_tensor *query_out, const rope_tensor *key_out,
                               void *stream);

/* Text describing the last failing call on the calling thread ("" if none).  The pointer
 * stays valid until the next call on this thread. */
const char *rope_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_AMD_H */
