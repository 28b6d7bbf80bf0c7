// bench_ceiling.hip -- measurement kernels for bench.py (not part of the RoPE library).
//
// Reference streams that do no arithmetic, built in the way the RoPE kernels stream (16-byte
// lanes, one item per lane, non-temporal loads; stores as the kernel they stand beside issues
// them), to put a measured ceiling beside each kernel's time:
//   ceiling_copy   a dense copy of `bytes` bytes: the attainable rate of a mixed read/write
//                  stream, and a copy of known size for scaling the HBM byte counters.  It
//                  runs one 16-byte vector per lane in one-wavefront workgroups and one pass,
//                  storing with the sc1 and nt cache bits: of the forms measured on MI355X (64-
//                  to 1024-lane workgroups, 1 to 8 vectors per lane, grid-stride loops of 2 to
//                  8 passes, persistent grids, per-XCD contiguous ranges, cached or streamed
//                  accesses, every combination of the sc0, sc1 and nt bits on loads and
//                  stores, loads and stores held to alternating time slots), this one copies
//                  85 MB to 1 GiB fastest (nt-only stores: 1-2% slower);
//   ceiling_rows   an in-place pass over a strided slice of each row (read `len` bytes at
//                  `off` of each `row_bytes`-byte row in lanes of `lane_bytes` (8 or 16), a lane
//                  taking its chunk in `rows_per_lane` consecutive rows (1, 2 or 4), write them
//                  back unchanged) plus dense side reads per row (`side_bytes` from each of two
//                  arrays, row r using side row r / rows_per_side, split evenly over the row's
//                  lanes in 16-byte loads, loaded once per lane): the access pattern of the
//                  in-place RoPE kernel on a [rows, D] slice with its cos/sin rows, with the
//                  rotation taken out (non-temporal stores, as that kernel's).
//   ceiling_pairs  a copy of `heads` rows of `head_bytes` in the cache kernel's NeoX pair-unit
//                  layout: a lane takes 16 bytes at u*16 of a head and 16 bytes half a head
//                  further (head_bytes / 32 lanes per head, all of a wavefront's lanes on
//                  whole heads), in `rows_per_lane` rows of heads (1 or 2), 256-lane
//                  workgroups, stores with the sc1 and nt bits as the cache kernel's; with the
//                  rotation and the cos|sin gather taken out.
// Each returns 0, or -1 for arguments outside their documented form and -2 if the launch
// fails.  Everything is enqueued on `stream` (a hipStream_t, NULL = the null stream).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int64_t kMaxGrid = int64_t(1) << 20;

// The dense copy: one wavefront per workgroup, one vector per lane; the grid covers the copy in
// one pass up to kCopyMaxGrid workgroups (32 GiB) and loops beyond.
constexpr int kCopyBlock = 64;
constexpr int64_t kCopyMaxGrid = int64_t(1) << 25;

// Stores as the cache kernel issues them: buffer stores with the device-scope and streaming
// cache bits (sc1 | nt), into a buffer range that starts at a wave-uniform base.
constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, no swizzle, no index stride
constexpr int kStoreSc1Nt = 16 | 2;

__device__ __forceinline__ void store_sc1nt(void *base, int64_t range_bytes, int off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      v, __builtin_amdgcn_make_buffer_rsrc(base, 0, int(range_bytes), kRsrcWord3), off, 0,
      kStoreSc1Nt);
}

__global__ __launch_bounds__(kCopyBlock) void copy_kernel(u32x4 *dst, const u32x4 *src,
                                                          int64_t n) {
  // ib: the first vector of this workgroup's pass (uniform), so the store range is scalar
  for (int64_t ib = int64_t(blockIdx.x) * kCopyBlock; ib < n;
       ib += int64_t(gridDim.x) * kCopyBlock) {
    const int64_t i = ib + threadIdx.x, left = n - ib;
    if (i < n)
      store_sc1nt(dst + ib, (left < kCopyBlock ? left : kCopyBlock) * 16, int(threadIdx.x) * 16,
                  __builtin_nontemporal_load(src + i));
  }
}

// One lane: W bytes (8 or 16) of the slice in each of R consecutive rows (rows that share one
// side row), and its share of that side row (16-byte loads from each side array, loaded once for
// the R rows).  `flip` is zero at run time; folding it into the data keeps every word of the
// stores live.  SIDE: 0 no side arrays, 1 cached side loads, 2 non-temporal ones.  The cache
// policy of every access is fixed per instantiation (the stores are buffer stores with the nt
// bit as an operand: with plain non-temporal stores the compiler merged the store paths and
// dropped the bit).  Item decode as cheap as the RoPE kernel's: shifts when the lanes of a row
// and the row groups of a side row are powers of two (every pattern the benchmark times), 32-bit
// division otherwise; lshift/sshift < 0 selects the division.
template <int W, int R, int SIDE>
__global__ __launch_bounds__(1024) void rows_kernel(char *x, uint32_t x_bytes, uint32_t lanes,
                                                    int64_t row_bytes, int64_t off,
                                                    uint32_t lanes_per_row, int lshift,
                                                    const char *side_a, const char *side_b,
                                                    int64_t side_bytes, uint32_t per_lane,
                                                    uint32_t groups_per_side, int sshift,
                                                    uint32_t flip) {
  using V = typename std::conditional<W == 16, u32x4, u32x2>::type;
  // per_lane: the side bytes each lane loads from each side row, a multiple of 16 (host)
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(x, 0, int(x_bytes), kRsrcWord3);
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t it = blockIdx.x * blockDim.x + threadIdx.x; it < lanes; it += stride) {
    const uint32_t g = lshift >= 0 ? it >> lshift : it / lanes_per_row;
    const uint32_t c = it - g * lanes_per_row;
    const int64_t o = int64_t(g) * R * row_bytes + off + int64_t(c) * W;  // below x_bytes
    V v[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const V *>(x + o + j * row_bytes));
    uint32_t acc = 0;
    if constexpr (SIDE != 0) {
      const uint32_t sr = sshift >= 0 ? g >> sshift : g / groups_per_side;  // the side row
      const int64_t so = int64_t(sr) * side_bytes + int64_t(c) * per_lane;
      uint32_t k = 0;
      do {
        const u32x4 *qa = reinterpret_cast<const u32x4 *>(side_a + so + k);
        const u32x4 *qb = reinterpret_cast<const u32x4 *>(side_b + so + k);
        const u32x4 a = SIDE == 2 ? __builtin_nontemporal_load(qa) : *qa;
        const u32x4 b = SIDE == 2 ? __builtin_nontemporal_load(qb) : *qb;
        acc |= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
        k += 16;
      } while (k < per_lane);
    }
    const uint32_t m = flip & acc;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      v[j].x ^= m;
      v[j].y ^= m;
      const int os = int(o + j * row_bytes);
      if constexpr (W == 16) {
        v[j].z ^= m;
        v[j].w ^= m;
        __builtin_amdgcn_raw_buffer_store_b128(v[j], rx, os, 0, 2);
      } else {
        __builtin_amdgcn_raw_buffer_store_b64(v[j], rx, os, 0, 2);
      }
    }
  }
}

// Lane l of a wavefront owns unit u = l % units of head l / units, in each of K rows of
// `hpw` heads; wavefront w covers heads [w*K*hpw, (w+1)*K*hpw).  Lanes past the last head
// copy nothing.
template <int K>
__global__ __launch_bounds__(256) void pairs_kernel(u32x4 *dst, const u32x4 *src, int64_t heads,
                                                   int64_t units, int64_t hpw, int64_t waves) {
  const int64_t lane = threadIdx.x & 63, hsub = lane / units, u = lane - hsub * units;
  const int64_t vpr = 2 * units;  // 16-byte vectors per head
  const int64_t w0 = __builtin_amdgcn_readfirstlane(int(blockIdx.x * 4 + threadIdx.x / 64));
  for (int64_t w = w0; w < waves; w += int64_t(gridDim.x) * 4) {
    // the wavefront's heads [h0, h0 + nh) as one store range
    const int64_t h0 = w * K * hpw, hl = heads - h0, nh = hl < K * hpw ? hl : K * hpw;
    u32x4 a[K], b[K];
    int64_t base[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      int64_t h = (w * K + k) * hpw + hsub;
      h = (hsub < hpw && h < heads) ? h : heads - 1;  // idle lanes reload the last head
      base[k] = h * vpr + u;
      a[k] = __builtin_nontemporal_load(src + base[k]);
      b[k] = __builtin_nontemporal_load(src + base[k] + units);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t h = (w * K + k) * hpw + hsub;
      if (hsub >= hpw || h >= heads) continue;
      const int off = int((base[k] - h0 * vpr) * 16);
      store_sc1nt(dst + h0 * vpr, nh * vpr * 16, off, a[k]);
      store_sc1nt(dst + h0 * vpr, nh * vpr * 16, off + int(units) * 16, b[k]);
    }
  }
}


bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" __attribute__((visibility("default"))) int ceiling_copy(void *dst, const void *src,
                                                                   int64_t bytes, void *stream) {
  if (!dst || !src || bytes <= 0 || bytes % 16 || !aligned(dst, 16) || !aligned(src, 16))
    return -1;
  const int64_t n = bytes / 16;
  int64_t grid = (n + kCopyBlock - 1) / kCopyBlock;
  grid = grid > kCopyMaxGrid ? kCopyMaxGrid : grid;
  hipLaunchKernelGGL(copy_kernel, dim3(uint32_t(grid)), dim3(kCopyBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4 *>(dst),
                     static_cast<const u32x4 *>(src), n);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" __attribute__((visibility("default"))) int ceiling_rows(
    void *x, int64_t rows, int64_t row_bytes, int64_t off, int64_t len, int64_t lane_bytes,
    int64_t rows_per_lane, const void *side_a, const void *side_b, int64_t side_bytes,
    int64_t rows_per_side, int side_stream, void *stream) {
  const int64_t w = lane_bytes, r = rows_per_lane;
  if (!x || (w != 8 && w != 16) || (r != 1 && r != 2 && r != 4) || rows <= 0 || rows % r ||
      len <= 0 || len % w || off % w || row_bytes % w || off + len > row_bytes ||
      !aligned(x, uintptr_t(w)) || rows_per_side <= 0 || rows_per_side % r || side_bytes < 0)
    return -1;
  const int64_t lanes_per_row = len / w;
  if (side_bytes % (16 * lanes_per_row) != 0) return -1;
  if (side_bytes > 0 && (!side_a || !side_b || !aligned(side_a, 16) || !aligned(side_b, 16)))
    return -1;
  const int64_t groups = rows / r, lanes = groups * lanes_per_row, x_bytes = rows * row_bytes;
  if (lanes >= (int64_t(1) << 31) || x_bytes >= (int64_t(1) << 31))
    return -1;  // 32-bit item decode and store offsets
  // the in-place RoPE kernel's launch shape: within one round of resident lanes (256 CUs x
  // 2048) the largest workgroup from 1024 down to 64 lanes that still gives every CU one,
  // 512-lane workgroups past it
  int64_t bl = 1024;
  while (bl > 64 && lanes < 256 * bl) bl /= 2;
  if (lanes > int64_t(256) * 2048) bl = 512;
  int64_t nb = (lanes + bl - 1) / bl;
  nb = nb < 1 ? 1 : (nb > kMaxGrid ? kMaxGrid : nb);
  const auto log2_exact = [](int64_t v) {
    int k = 0;
    while ((int64_t(1) << k) < v) ++k;
    return (int64_t(1) << k) == v ? k : -1;
  };
  const int64_t gps = rows_per_side / r;  // row groups per side row
  const int lsh = log2_exact(lanes_per_row), ssh = log2_exact(gps);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char *a = static_cast<const char *>(side_a), *b = static_cast<const char *>(side_b);
  const dim3 grid(static_cast<uint32_t>(nb)), block(static_cast<uint32_t>(bl));
  char *xc = static_cast<char *>(x);
#define ROWS_LAUNCH(W, R, SIDE)                                                              \
  hipLaunchKernelGGL((rows_kernel<W, R, SIDE>), grid, block, 0, s, xc, uint32_t(x_bytes),     \
                     uint32_t(lanes), row_bytes, off, uint32_t(lanes_per_row), lsh, a, b,      \
                     side_bytes, uint32_t(side_bytes / lanes_per_row), uint32_t(gps), ssh, 0u)
#define ROWS_SIDE(W, R)                                                                      \
  do {                                                                                       \
    if (side_bytes == 0) ROWS_LAUNCH(W, R, 0);                                               \
    else if (side_stream) ROWS_LAUNCH(W, R, 2);                                              \
    else ROWS_LAUNCH(W, R, 1);                                                               \
  } while (0)
  if (w == 16) {
    if (r == 1) ROWS_SIDE(16, 1);
    else if (r == 2) ROWS_SIDE(16, 2);
    else ROWS_SIDE(16, 4);
  } else {
    if (r == 1) ROWS_SIDE(8, 1);
    else if (r == 2) ROWS_SIDE(8, 2);
    else ROWS_SIDE(8, 4);
  }
#undef ROWS_SIDE
#undef ROWS_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" __attribute__((visibility("default"))) int ceiling_pairs(void *dst, const void *src,
                                                                    int64_t heads,
                                                                    int64_t head_bytes,
                                                                    int64_t rows_per_lane,
                                                                    void *stream) {
  if (!dst || !src || heads <= 0 || head_bytes <= 0 || head_bytes % 32 ||
      head_bytes / 32 > 64 || (rows_per_lane != 1 && rows_per_lane != 2) || !aligned(dst, 16) ||
      !aligned(src, 16))
    return -1;
  const int64_t units = head_bytes / 32, hpw = 64 / units;
  const int64_t per_wave = hpw * rows_per_lane, waves = (heads + per_wave - 1) / per_wave;
  int64_t blocks = (waves + 3) / 4;
  blocks = blocks > kMaxGrid ? kMaxGrid : blocks;
  hipStream_t s = static_cast<hipStream_t>(stream);
  u32x4 *d = static_cast<u32x4 *>(dst);
  const u32x4 *c = static_cast<const u32x4 *>(src);
  if (rows_per_lane == 1)
    hipLaunchKernelGGL(pairs_kernel<1>, dim3(uint32_t(blocks)), dim3(256), 0, s, d, c, heads,
                       units, hpw, waves);
  else
    hipLaunchKernelGGL(pairs_kernel<2>, dim3(uint32_t(blocks)), dim3(256), 0, s, d, c, heads,
                       units, hpw, waves);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
