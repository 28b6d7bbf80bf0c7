// rope_plan.h -- host-side launch plans shared by the validation code and the HIP launchers
// of librope_amd.so (library-internal; not part of the C ABI).
#pragma once

#include <cstdint>
#include <string>

#include "rope.h"

namespace ropeamd {

// Division of a 32-bit unsigned dividend by a run-time invariant divisor, done as a
// multiply-high, an add and two shifts (Granlund & Montgomery, "Division by Invariant
// Integers using Multiplication", PLDI 1994, the round-up method for N = 32).
//   l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
//   q = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0) with t = mulhi(m, n).
struct FastDiv {
  uint32_t d = 1, m = 1, s1 = 0, s2 = 0;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

// Host evaluation of the same formula (used by the CPU tests of the plan logic).
inline uint32_t fastdiv_host(const FastDiv &f, uint32_t n) {
  uint32_t t = uint32_t((uint64_t(f.m) * n) >> 32);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

// ---- in-place partial RoPE ----------------------------------------------------------------
// Interleave mode: the slice of every row (b, s, n) is cut into `chunks_per_row` chunks of
// `vec` elements; one GPU lane owns one chunk (all pairs of a chunk are lane-local because
// vec is even and chunks start at even offsets from the slice start).  Half mode: the first
// half of the slice is cut into chunks; the lane owning chunk u also owns chunk u of the
// second half, which holds the partners (i + L/2) of its elements.  When cos/sin are shared
// by the heads of a (b, s) (broadcast over N), a lane owns that chunk of `nhl` consecutive
// heads and loads the cos/sin chunk once for all of them.
struct InplacePlan {
  bool half = false;  // rotary_mode 0
  // Half mode with pairs split across lanes: each lane owns one chunk of one half, and its
  // partner chunk (same position in the other half) belongs to lane (lane ^ xch), fetched by a
  // cross-lane read.  xch is the chunk count of a half rounded up to a power of two, at most
  // 16, so a row's 2 * xch lanes never straddle a wavefront.  0 = the lane owns both chunks.
  uint32_t xch = 0;
  // chunks of one half (<= xch; xch is the next power of two): a row's lanes u with
  // u % xch >= xch_cph carry no chunk (they load the half's last chunk and store nothing)
  uint32_t xch_cph = 0;
  uint32_t nhl = 1;   // heads per lane (1, 2 or 4); > 1 only when cos/sin broadcast over N
  rope_dtype xdt = ROPE_F32, cdt = ROPE_F32;
  bool vector_io = false;  // 16-byte x accesses (else one element at a time)
  bool noop = false;       // nothing to launch
  void *x = nullptr;
  const void *cos = nullptr, *sin = nullptr;
  int64_t B = 0, S = 0, N = 0, D = 0, start = 0, L = 0;
  int64_t rows = 0;             // B*S*N
  int64_t items = 0;            // (rows / nhl) * chunks_per_row
  uint32_t vec = 2;             // elements per lane chunk
  uint32_t chunks_per_row = 0;  // L / vec (half mode: (L/2) / vec)
  // cos/sin row of x-row (b, s, n) = b*cb + s*cs + n*cn (in rows of L elements)
  int64_t cb = 0, cs = 0, cn = 0;
  bool cos_stream = false;  // every cos/sin row is read by exactly one lane group (streamed)
  bool idx32 = true;  // items, N / nhl, S and nhl * D fit in 32 bits: use FastDiv below
  FastDiv div_cpr, div_ng;  // by chunks_per_row, N / nhl
  uint32_t block = 1024;  // workgroup size: kBlock, or kBlockMulti past one round of lanes
  // The cos/sin row of row group r = (b*S + s)*ng + g (ng = N / nhl), written without
  // decoding b, s and g:  b*cb + s*cs + g*nhl*cn = r*crow_a + (r / ng)*crow_b + (r / (ng*S))*crow_c
  // (as g = r - ng*(r/ng), s = r/ng - S*(r/(ng*S)) and b = r/(ng*S)).  The coefficients are
  // taken mod 2^32 (crow_b and crow_c may be negative); the row itself is below 2^31 wherever
  // the 32-bit item loop runs.  A zero coefficient skips its division: per-head tables, and
  // tables shared over N when a row holds one head group, need none; tables shared by several
  // head groups of a (b, s) need one.
  uint32_t crow_a = 0, crow_b = 0, crow_c = 0;
  FastDiv div_ngs;  // by ng * S
};

// ---- cos/sin cache --------------------------------------------------------------------------
// A workgroup owns a tile of `tile_tokens` tokens.  It first stages the tile's cos|sin rows
// (gathered, mrope-stitched, in the cache's element type) in LDS, then its lanes walk the tile's
// (token, head, unit) items.  NeoX: a unit is two vectors of `vec` elements (vector u and
// vector u + rd/(2 vec) of the rotated part, or the same shape over the pass-through part).
// GPT-J: a unit is one vector.
struct CachePlan {
  rope_dtype dt = ROPE_F32;
  bool neox = true;
  bool mrope = false;
  bool interleaved = false;  // cacheMode 1: rows 1 and 2 take the elements 1, 4, ... / 2, 5, ...
  bool multi_row = false;    // some staging chunk draws on more than one position row
  int32_t interleave_end = 0;  // 3 * mropeSection[1]: end of the interleaved elements
  bool vector_io = false;
  const int64_t *positions = nullptr;
  const void *q_in = nullptr, *k_in = nullptr, *cache = nullptr;
  void *q_out = nullptr, *k_out = nullptr;
  int64_t T = 0, nq = 0, nk = 0, H = 0, rd = 0, max_seq = 0;
  int64_t q_stride = 0, k_stride = 0, cache_stride = 0;  // row strides in elements
  int64_t pos_stride_row = 0, pos_stride_tok = 0;        // positions[k, t] strides
  int32_t sec_end[4] = {0, 0, 0, 0};  // cumulative mrope section ends (in cos/sin index)
  int32_t nsec = 0;
  uint32_t vec = 1;          // elements per vector
  uint32_t units = 0;        // units per head (NeoX H / (2 vec), GPT-J H / vec)
  uint32_t rot_units = 0;    // rotated units per head (NeoX rd / (2 vec), GPT-J rd / vec)
  uint32_t items_per_token = 0;
  uint32_t tile_tokens = 1;
  int64_t tiles = 0;
  // Tapered end: tiles [0, big_tiles) hold tile_tokens tokens each (tokens [0, big_tokens));
  // every later tile holds one token, so the workgroups of the last round are short.
  int64_t big_tiles = 0, big_tokens = 0;
  bool cache_vec = false;       // cache rows can be read with 16-byte loads
  // rope mode with rotaryDim > 16384 (a cos|sin row beyond the 64 KiB LDS tile): no staging;
  // every item reads its cos/sin chunk from its token's cache row
  bool cs_direct = false;
  uint32_t stage_chunks = 0;    // (rd/2) / vec: vector chunks of one cos (or sin) half-row
  FastDiv div_units, div_ipt, div_stage;
  // Wavefront path (cos_sin_cache_wave_kernel): one wavefront per (token, group of heads), no
  // LDS.  Lane l owns unit l % units of head l / units of each of wave_rows rows of wave_hpw
  // heads, so its cos|sin chunk is the same for all its items and is read straight from the
  // cache row.  Lanes from wave_hpw * units up are idle.
  bool wave = false;
  uint32_t wave_hpw = 0;        // heads per row of 64 lanes: floor(64 / units)
  uint32_t wave_heads = 0;      // heads per wavefront: wave_rows * wave_hpw
  uint32_t wave_wpt = 0;        // wavefronts per token: ceil((nq + nk) / wave_heads)
  int64_t waves = 0;            // T * wave_wpt (< 2^31)
  FastDiv div_wpt;
  // NeoX with rotaryDim <= headSize / 2: a lane's two accesses take vectors u and units + u of
  // the head (whole lines per access); a rotated vector's pair partner comes from another
  // lane of the same head (cross-lane read)
  bool wave_xch = false;
  // NeoX with one-vector units (a head's vectors on consecutive lanes, 2 * units lanes per
  // head); rotated pairs are completed by the same cross-lane read
  bool wave_lin = false;
  // head rows per lane: kWaveRowsPairUnits (NeoX pair units without multi-row stitching) or
  // kWaveRowsVectorUnits; the kernel has it as a template argument (last in the struct, so
  // the fields the kernels read keep their offsets)
  uint32_t wave_rows = 0;
  uint32_t wave_block = 0;      // lanes per workgroup: kWaveBlockNeox or kWaveBlockGptj
  // GPT-J rope mode with a 128-byte cos|sin row, in a launch of at least kScalarRowMinWaves
  // wavefronts: each wavefront reads its token's whole row with two scalar loads, and each
  // lane selects its chunk from those registers (no vector loads for cos/sin)
  bool wave_scalar_row = false;
};

int plan_inplace(const rope_tensor *x, const rope_tensor *cos, const rope_tensor *sin,
                 int64_t rotary_mode, const int64_t *partial_slice, int64_t partial_slice_len,
                 InplacePlan *plan, std::string *err);

int plan_cache(const rope_tensor *positions, const rope_tensor *query_in,
               const rope_tensor *key_in, const rope_tensor *cos_sin_cache,
               const int64_t *mrope_section, int64_t mrope_section_len, int64_t head_size,
               int is_neox_style, int64_t cache_mode, const rope_tensor *query_out,
               const rope_tensor *key_out, CachePlan *plan, std::string *err);

// Workgroup size and the work units (16-byte chunks / two-vector units) a lane carries per
// pass.  Few units per lane and many waves keep more independent HBM requests in flight on
// gfx950 than deep per-lane unrolling.
// In-place kernel workgroups.  A launch that fits one round of resident lanes (256 CUs x
// 2048 lanes) takes the largest of kBlock, kBlock/2, ... 64 lanes that still gives every CU a
// workgroup: large workgroups dispatch faster, but a small launch in a few large workgroups
// funnels all its traffic through a few CUs.  A longer launch takes kBlockMulti, whose slots
// free up and refill sooner once waves start to finish at different times.
constexpr int64_t kComputeUnits = 256;  // MI355X
constexpr int kBlock = 1024;
constexpr int kBlockMulti = 512;
constexpr int kBlockMin = 64;
constexpr int64_t kOneRoundLanes = kComputeUnits * 2048;
// Cache kernel: with no more tokens than one round of resident workgroups (256 CUs x 7),
// every token gets a tile of its own, so each workgroup's chain of dependent memory round
// trips is as short as it can be.
constexpr int64_t kOneRoundCacheTiles = kComputeUnits * 7;
// Most workgroups in one launch; both kernels loop over the rest of the work.
constexpr int64_t kMaxGrid = int64_t(1) << 20;
constexpr int kCacheBlock = 256;  // cache kernel workgroup (one token tile)
// Tokens given one-token tiles at the end of a cache launch (about two thirds of a round of
// resident cache workgroups on MI355X, 256 CUs x 7; measured against 640, 2560 and 4096).
constexpr int64_t kTaperTokens = 1280;
constexpr int kNeoxItemsPerLane = 2;  // NeoX units are two vectors
constexpr int kGptjItemsPerLane = 2;  // GPT-J units are one vector
// Wavefront cache kernel: workgroups of independent wavefronts, 64 lanes for GPT-J and 256
// for the NeoX layouts.  GPT-J with 64-lane workgroups: 1-2.5% faster on five of seven shapes
// (the 1 GiB f16 one 1.1%), 0.5-0.8% slower on two; the NeoX layouts were up to 1% slower with
// them, and 128-, 512- and 1024-lane workgroups were slower still (up to 8%).  A lane carries
// two 16-byte q/k vectors per wavefront: NeoX pair units (two vectors each) one head row, the
// one-vector units of the other layouts two head rows.  Measured on the rope NeoX bf16, GPT-J
// f16 and mrope bf16 workloads: one-vector units with one row were 3-30% slower and with three
// rows 2-6% slower; pair units with one row 3% faster than with two, except under multi-row
// stitching (three cos|sin gathers per lane), where one row was 2-3% slower.
constexpr int kWaveBlockNeox = 256;
constexpr int kWaveBlockGptj = 64;
// The scalar cos|sin row: on the 1 GiB GPT-J f16 workload (rotaryDim 64 of 128) 2.2% faster
// than the two vector loads per lane, other GPT-J shapes with 128-byte rows 0.6-2.5%; at 64
// tokens (512 wavefronts) 6% slower, where the extra scalar round trip is not hidden.  Taken
// from eight wavefronts per compute unit up.
constexpr int64_t kScalarRowBytes = 128;
constexpr int64_t kScalarRowMinWaves = int64_t(kComputeUnits) * 8;
constexpr uint32_t kWaveRowsPairUnits = 1;
constexpr uint32_t kWaveRowsVectorUnits = 2;
// Waves of one launch stay below 2^31, so a wave index plus the grid stride fits 32 bits.
constexpr int64_t kMaxWaves = (int64_t(1) << 31) - (int64_t(1) << 24);

}  // namespace ropeamd
