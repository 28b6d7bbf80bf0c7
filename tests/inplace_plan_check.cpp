// Host check of the in-place op's launch plan (rope_plan.cpp) together with the work-item
// decode that inplace_rope_kernel applies to it, written out here for the host.  For each
// plan it walks every work item exactly as a lane would and checks that
//   - every element of every row's slice [start, end) is read and written by exactly one
//     item, and nothing outside the slices is touched;
//   - the cos/sin element each x element is paired with is the one of its own (b, s, n) row
//     (broadcast dims give index 0) at the same slice position, inside the cos/sin tensor;
//   - in half mode an item's two chunks lie L/2 apart in one row; or, when the plan splits a
//     pair across lanes (xch), the item it ^ xch -- the lane it ^ xch of the same wavefront --
//     holds the same row's chunk L/2 away, and a row's lanes never straddle a wavefront.
// Shapes cover both modes, every dtype pair, every broadcast layout, aligned and unaligned
// pointers (vector and element paths) and 1/2/4 heads per lane.  Every plan's workgroup size
// follows its launch length, and a 32-bit plan's item index plus the grid stride never wraps;
// plans of 2^31, 2^31 + 128 and 3 * 2^30 items sit either side of the 32-bit limit, and a plan
// with 2^32 items is checked for taking the 64-bit decode, with sampled items in bounds.  No GPU and no
// tensor data are involved: descriptors carry made-up, suitably aligned addresses.
// Prints "ok <plans> <items>" or the first failure; exit status 1 on failure.
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "rope.h"
#include "rope_plan.h"

using namespace ropeamd;

static rope_tensor desc(uintptr_t addr, rope_dtype dt, int64_t B, int64_t S, int64_t N,
                        int64_t D) {
  rope_tensor t{};
  t.data = reinterpret_cast<void *>(addr);
  t.dtype = dt;
  t.ndim = 4;
  const int64_t sh[4] = {B, S, N, D};
  int64_t st = 1;
  for (int d = 3; d >= 0; --d) {
    t.shape[d] = sh[d];
    t.stride[d] = st;
    st *= sh[d];
  }
  return t;
}

static int esize(rope_dtype dt) { return dt == ROPE_F32 ? 4 : 2; }

// The decode of inplace_rope_kernel: item -> (r, chunk) and the cos/sin row of r, then the
// first x element and the first cos/sin element of the item's chunk.  The 32-bit decode takes
// the cos/sin row from the plan's coefficients (arithmetic mod 2^32, skipping the divisions
// of zero coefficients), as the kernel does; the 64-bit one from (b, s, g).  (b, s, g) are
// also decoded here by plain division, for the range checks.
struct Decoded {
  uint64_t r, chunk, b, s, g;
  int64_t crow;
};

static Decoded decode(const InplacePlan &p, uint64_t it) {
  Decoded d{};
  const uint64_t ng = uint64_t(p.N) / p.nhl;
  if (p.idx32) {
    const uint32_t i32 = uint32_t(it);
    const uint32_t r = fastdiv_host(p.div_cpr, i32);
    d.r = r;
    d.chunk = i32 - r * p.chunks_per_row;
    uint32_t crow = r * p.crow_a;
    if (p.crow_b != 0) crow += fastdiv_host(p.div_ng, r) * p.crow_b;
    if (p.crow_c != 0) crow += fastdiv_host(p.div_ngs, r) * p.crow_c;
    d.crow = int64_t(crow);
  } else {
    d.r = it / p.chunks_per_row;
    d.chunk = it - d.r * p.chunks_per_row;
  }
  const uint64_t bs = d.r / ng;
  d.g = d.r - bs * ng;
  d.b = bs / uint64_t(p.S);
  d.s = bs - d.b * uint64_t(p.S);
  if (!p.idx32) d.crow = int64_t(d.b) * p.cb + int64_t(d.s) * p.cs + int64_t(d.g) * p.nhl * p.cn;
  return d;
}

static int fails = 0;
static uint64_t items_checked = 0;
static int padded_plans = 0;

#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      if (fails++ == 0) {                                 \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
        std::printf(__VA_ARGS__);                         \
        std::printf("\n");                                \
      }                                                   \
      return false;                                       \
    }                                                     \
  } while (0)

// Full coverage walk of one plan.
static bool walk(int64_t B, int64_t S, int64_t N, int64_t D, int64_t start, int64_t end,
                 int64_t Bc, int64_t Sc, int64_t Nc, rope_dtype xdt, rope_dtype cdt, int mode,
                 uintptr_t xoff_bytes) {
  const rope_tensor x = desc(0x10000000 + xoff_bytes, xdt, B, S, N, D);
  const int64_t L = end - start;
  const rope_tensor c = desc(0x90000000, cdt, Bc, Sc, Nc, L);
  const rope_tensor sn = desc(0xA0000000, cdt, Bc, Sc, Nc, L);
  const int64_t sl[2] = {start, end};
  InplacePlan p;
  std::string err;
  const int st = plan_inplace(&x, &c, &sn, mode, sl, 2, &p, &err);
  CHECK(st == ROPE_OK, "plan rejected: %s", err.c_str());
  if (p.noop) return true;
  if (p.xch && p.xch_cph < p.xch) ++padded_plans;
  const int64_t V = p.vec, NHL = p.nhl, NH = (p.half && !p.xch) ? 2 : 1;
  const int64_t hoff = p.half ? L / 2 : 0;
  CHECK(p.xch == 0 || (p.half && p.vector_io && (p.xch & (p.xch - 1)) == 0 && p.xch <= 16 &&
                       p.xch_cph <= p.xch && 2 * p.xch_cph > p.xch &&
                       p.chunks_per_row == 2 * p.xch && int64_t(p.xch_cph) * V == L / 2),
        "lane exchange with xch %u (%u chunks per half), chunks %u, V %lld, L %lld", p.xch,
        p.xch_cph, p.chunks_per_row, (long long)V, (long long)L);
  CHECK(!p.idx32 || uint64_t(p.items) - 1 + uint64_t(kMaxGrid) * p.block < (uint64_t(1) << 32),
        "32-bit item index can wrap: items %lld, block %u", (long long)p.items, p.block);
  // the 32-bit loop forms its offsets as 32 x 32 -> 64-bit products of r with nhl * D, and of
  // the cos/sin row with L
  CHECK(!p.idx32 || (uint64_t(p.nhl) * uint64_t(D) < (uint64_t(1) << 32) &&
                     uint64_t(L) < (uint64_t(1) << 32)),
        "32-bit plan with nhl * D = %llu", (unsigned long long)(p.nhl * D));
  {
    // the largest power-of-two workgroup (1024 down to 64) that gives each CU one, or 512
    // lanes past one round of resident lanes
    uint32_t want = 1024;
    while (want > 64 && uint64_t(p.items) < 256ull * want) want /= 2;
    if (p.items > int64_t(256) * 2048) want = 512;
    CHECK(p.block == want, "workgroup of %u lanes for %lld items, want %u", p.block,
          (long long)p.items, want);
  }
  CHECK(NHL == 1 || (p.vector_io && NHL * NH * V * esize(xdt) <= 32),
        "heads per lane %lld with %lld x bytes per head: no kernel is built for it",
        (long long)NHL, (long long)(NH * V * esize(xdt)));
  CHECK(NHL == 1 || (Nc == 1 && N % NHL == 0), "heads per lane %lld with Nc %lld N %lld",
        (long long)NHL, (long long)Nc, (long long)N);
  // items carrying a chunk (all of them, except the lanes past a half's last chunk in XCH)
  const uint64_t owning = p.xch ? uint64_t(p.items) / (2 * p.xch) * (2 * p.xch_cph)
                                : uint64_t(p.items);
  CHECK(owning * NHL * NH * V == uint64_t(B * S * N * L),
        "items %lld do not tile the slices", (long long)p.items);
  std::vector<uint8_t> hit(size_t(B * S * N * D), 0);
  for (uint64_t it = 0; it < uint64_t(p.items); ++it) {
    const Decoded d = decode(p, it);
    CHECK(d.b < uint64_t(B) && d.s < uint64_t(S) && d.g * NHL < uint64_t(N) &&
              d.chunk < p.chunks_per_row,
          "item %llu decodes out of range", (unsigned long long)it);
    const int64_t crow = d.crow;
    // the kernel's element offset of a chunk (XCH: half, then chunk of the half; a lane past
    // a half's last chunk loads that chunk and stores nothing)
    auto elem_of = [&](uint64_t chunk, bool *owns) {
      if (!p.xch) {
        *owns = true;
        return int64_t(chunk) * V;
      }
      const uint32_t c = uint32_t(chunk) & (p.xch - 1);
      *owns = c < p.xch_cph;
      return (chunk >= p.xch ? L / 2 : 0) + int64_t(*owns ? c : p.xch_cph - 1) * V;
    };
    bool owns;
    const int64_t elem = elem_of(d.chunk, &owns);
    const int64_t coff = crow * L + elem;
    const int64_t x0 = int64_t(d.r) * NHL * D + start + elem;
    if (p.xch) {
      const Decoded q = decode(p, it ^ p.xch);
      CHECK(q.r == d.r && q.chunk == (d.chunk ^ p.xch) && (it & 63) / (2 * p.xch) ==
                                                              ((it ^ p.xch) & 63) / (2 * p.xch),
            "item %llu and its partner lane are not the pair chunks of one row",
            (unsigned long long)it);
      bool q_owns;
      const int64_t xq = int64_t(q.r) * NHL * D + start + elem_of(q.chunk, &q_owns);
      CHECK(q_owns == owns, "item %llu and its partner lane disagree on carrying a chunk",
            (unsigned long long)it);
      CHECK(xq - x0 == (d.chunk < p.xch ? hoff : -hoff), "partner chunk not L/2 away");
    }
    for (int64_t j = 0; j < NHL; ++j)
      for (int64_t hh = 0; hh < NH; ++hh)
        for (int64_t e = 0; e < V; ++e) {
          const int64_t xi = x0 + j * D + hh * hoff + e;
          const int64_t ci = coff + hh * hoff + e;
          CHECK(xi >= 0 && xi < B * S * N * D, "x index %lld out of bounds", (long long)xi);
          const int64_t row = xi / D, col = xi % D;
          CHECK(col >= start && col < end, "x index %lld outside the slice", (long long)xi);
          const int64_t n = row % N, bs = row / N, s = bs % S, b = bs / S;
          const int64_t want = (((Bc == 1 ? 0 : b) * Sc + (Sc == 1 ? 0 : s)) * Nc +
                                (Nc == 1 ? 0 : n)) * L + (col - start);
          CHECK(ci == want, "x (%lld,%lld,%lld,%lld) paired with cos %lld, want %lld",
                (long long)b, (long long)s, (long long)n, (long long)col, (long long)ci,
                (long long)want);
          CHECK(ci < Bc * Sc * Nc * L, "cos index out of bounds");
          if (!owns) continue;  // loads only
          CHECK(hit[size_t(xi)] == 0, "x index %lld touched twice", (long long)xi);
          hit[size_t(xi)] = 1;
        }
    ++items_checked;
  }
  for (int64_t i = 0; i < B * S * N * D; ++i) {
    const int64_t col = i % D;
    CHECK(hit[size_t(i)] == (col >= start && col < end ? 1 : 0),
          "x index %lld coverage %d", (long long)i, int(hit[size_t(i)]));
  }
  return true;
}

// cos/sin of the very large plans below sit 2^46 bytes up, clear of x's tens of GiB.
constexpr uintptr_t kFarTables = uintptr_t(1) << 46;

// Plans at the 32-bit limit: 2^31 items is the largest on the 32-bit decode; 2^31 + 128 and
// 3 * 2^30 items (where a 32-bit index plus the grid stride would wrap) take the 64-bit one.
static bool limits() {
  for (int64_t S : {int64_t(1) << 24, (int64_t(1) << 24) + 1, int64_t(3) << 23}) {
    const rope_tensor x = desc(0x10000000, ROPE_BF16, 1, S, 1, 1024);
    const rope_tensor c = desc(kFarTables, ROPE_BF16, 1, 1, 1, 1024);
    InplacePlan p;
    std::string err;
    CHECK(plan_inplace(&x, &c, &c, 1, nullptr, 0, &p, &err) == ROPE_OK, "%s", err.c_str());
    CHECK(p.items == S * 128 && p.idx32 == (p.items <= (int64_t(1) << 31)) &&
              p.block == uint32_t(kBlockMulti),
          "S %lld: items %lld idx32 %d block %u", (long long)S, (long long)p.items,
          int(p.idx32), p.block);
    CHECK(!p.idx32 || uint64_t(p.items) - 1 + uint64_t(kMaxGrid) * p.block < (uint64_t(1) << 32),
          "S %lld: 32-bit index can wrap", (long long)S);
  }
  return true;
}

// The 2^32-item plan: 64-bit decode, sampled items in bounds.
static bool huge() {
  const int64_t S = int64_t(1) << 25, D = 1024;
  const rope_tensor x = desc(0x10000000, ROPE_BF16, 1, S, 1, D);
  const rope_tensor c = desc(kFarTables, ROPE_BF16, 1, 1, 1, D);
  InplacePlan p;
  std::string err;
  CHECK(plan_inplace(&x, &c, &c, 1, nullptr, 0, &p, &err) == ROPE_OK, "%s", err.c_str());
  CHECK(!p.idx32 && uint64_t(p.items) == (uint64_t(1) << 32) && p.vec == 8 && p.nhl == 1,
        "huge plan: idx32 %d items %lld vec %u nhl %u", int(p.idx32), (long long)p.items,
        p.vec, p.nhl);
  uint64_t z = 0x9E3779B97F4A7C15ull;
  for (int k = 0; k < 100000; ++k) {
    z ^= z << 13; z ^= z >> 7; z ^= z << 17;
    const uint64_t it = k < 4 ? (k < 2 ? uint64_t(k) : uint64_t(p.items) - 1 - (k - 2))
                              : z % uint64_t(p.items);
    const Decoded d = decode(p, it);
    const int64_t x0 = int64_t(d.r) * D + int64_t(d.chunk) * 8;
    CHECK(d.s < uint64_t(S) && d.b == 0 && x0 >= 0 && x0 + 8 <= S * D, "item %llu",
          (unsigned long long)it);
    CHECK(x0 == int64_t(it) * 8, "item %llu maps to %lld", (unsigned long long)it,
          (long long)x0);
  }
  return true;
}

// The layouts that skip divisions in the kernel's cos/sin row: per-head tables and tables
// shared by one head group per row need none, tables shared by several head groups one (by
// the head groups per row); broadcast over B or S needs both.
static bool division_free() {
  struct Case {
    int64_t B, S, N, D, start, end, Bc, Sc, Nc;
    rope_dtype xdt;
    bool want_b, want_c;
  };
  const Case cases[] = {
      {8, 4096, 1, 576, 512, 576, 8, 4096, 1, ROPE_BF16, false, false},  // one head, BS1D
      {4, 2048, 32, 192, 128, 192, 4, 2048, 1, ROPE_BF16, true, false},  // 32 heads, BS1D
      {1, 524288, 2, 64, 0, 64, 1, 524288, 1, ROPE_F32, false, false},   // 2 heads on a lane
      {2, 16, 8, 128, 0, 128, 2, 16, 8, ROPE_BF16, false, false},        // BSND
      {2, 16, 8, 128, 0, 128, 1, 16, 8, ROPE_BF16, false, true},         // 1SND
      {2, 16, 8, 128, 0, 128, 2, 1, 8, ROPE_BF16, true, true},           // B1ND
  };
  for (const Case &k : cases) {
    const rope_tensor x = desc(0x10000000, k.xdt, k.B, k.S, k.N, k.D);
    const rope_tensor c = desc(0x90000000, ROPE_F32, k.Bc, k.Sc, k.Nc, k.end - k.start);
    const int64_t sl[2] = {k.start, k.end};
    InplacePlan p;
    std::string err;
    CHECK(plan_inplace(&x, &c, &c, 1, sl, 2, &p, &err) == ROPE_OK, "%s", err.c_str());
    CHECK(p.idx32 && (p.crow_b != 0) == k.want_b && (p.crow_c != 0) == k.want_c,
          "[%lld,%lld,%lld,%lld] cos [%lld,%lld,%lld]: coefficients %u %u %u",
          (long long)k.B, (long long)k.S, (long long)k.N, (long long)k.D, (long long)k.Bc,
          (long long)k.Sc, (long long)k.Nc, p.crow_a, p.crow_b, p.crow_c);
  }
  return true;
}

int main() {
  int plans = 0;
  const rope_dtype pairs[5][2] = {{ROPE_F32, ROPE_F32}, {ROPE_F16, ROPE_F16}, {ROPE_F16, ROPE_F32},
                                  {ROPE_BF16, ROPE_BF16}, {ROPE_BF16, ROPE_F32}};
  struct Shape { int64_t B, S, N, D, start, end; };
  const Shape shapes[] = {{2, 5, 8, 64, 0, 64},   {3, 4, 12, 96, 32, 96}, {2, 3, 6, 48, 16, 48},
                          {1, 7, 5, 40, 8, 40},   {2, 3, 2, 40, 1, 37},   {2, 2, 16, 24, 0, 16},
                          {1, 2, 40, 128, 64, 128}, {2, 3, 4, 10, 4, 6},  {1, 2, 3, 1024, 0, 1024},
                          {2, 3, 4, 48, 8, 20},
                          // half mode with chunk counts per half that are not powers of two
                          {2, 3, 4, 96, 0, 96},   {1, 3, 6, 128, 8, 104}, {2, 2, 3, 80, 0, 80},
                          {2, 3, 2, 64, 24, 64},  {3, 2, 2, 24, 0, 24}};
  for (const auto &sh : shapes)
    for (const auto &pr : pairs)
      for (int mode = 0; mode < 2; ++mode)
        for (int lay = 0; lay < 8; ++lay)
          for (uintptr_t mis : {uintptr_t(0), uintptr_t(2)}) {
            if (mis && pr[0] == ROPE_F32) continue;  // a 2-byte offset of an f32 tensor
            const int64_t Bc = (lay >= 4) ? 1 : sh.B;
            const int64_t Sc = (lay == 2 || lay == 3 || lay == 4 || lay == 7) ? 1 : sh.S;
            const int64_t Nc = (lay == 0 || lay == 2 || lay == 5 || lay == 7) ? sh.N : 1;
            // lay: 0 BSND, 1 BS1D, 2 B1ND, 3 B11D, 4 111D, 5 1SND, 6 1S1D, 7 11ND
            if (!walk(sh.B, sh.S, sh.N, sh.D, sh.start, sh.end, Bc, Sc, Nc, pr[0], pr[1], mode,
                      mis * esize(pr[0]) / 2))
              return 1;
            ++plans;
          }
  if (!limits() || !huge() || !division_free()) return 1;
  if (padded_plans == 0) {
    std::printf("FAIL: no half-mode plan pads its lane pairs\n");
    return 1;
  }
  std::printf("ok %d %llu (%d half-mode plans with padded lane pairs)\n", plans,
              (unsigned long long)items_checked, padded_plans);
  return 0;
}
