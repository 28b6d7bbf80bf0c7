// Host check of the cos/sin-cache op's launch plan (rope_plan.cpp) together with the way
// cos_sin_cache_kernel walks it, written out here for the host: tiles of tokens, the
// (token, head, unit) items of a tile and the cos|sin staging chunks.  For each plan it
// checks that
//   - every element of query_out and key_out is written by exactly one item, from the input
//     element at the same position of the same head (NeoX units pair elements i and
//     i + rotaryDim/2, GPT-J units hold whole pairs), and inputs are read inside their rows;
//   - the rotated part of each unit reads the cos|sin elements of its own pair indices;
//   - every token belongs to exactly one tile (tiles of tile_tokens, then one-token tiles),
//     and a launch of at most one round of workgroups (256 CUs x 7) has one-token tiles only;
//   - the staging lanes of a tile write each of its tile_tokens * rotaryDim LDS elements once,
//     inside the LDS size the launch requests, and each element's position row is the one the
//     stitching assigns (sections for cacheMode 0, the i mod 3 rule below 3 * mropeSection[1]
//     for cacheMode 1), with one row per chunk unless the plan takes the multi-row path (one
//     lane per chunk and row, writing that row's elements).
// Shapes cover every dtype, both styles, rope mode, every whitelisted mropeSection and both
// cacheModes, pass-through parts, token counts that leave a ragged last tile, reach the
// one-token tiles of the tapered end or sit either side of one round of workgroups, and
// padded row strides.  No GPU and no tensor data are
// involved.
// Prints "ok <plans> <items>" or the first failure; exit status 1 on failure.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "rope.h"
#include "rope_plan.h"

using namespace ropeamd;

static rope_tensor t2(uintptr_t addr, rope_dtype dt, int64_t rows, int64_t cols,
                      int64_t row_stride) {
  rope_tensor t{};
  t.data = reinterpret_cast<void *>(addr);
  t.dtype = dt;
  t.ndim = 2;
  t.shape[0] = rows;
  t.shape[1] = cols;
  t.stride[0] = row_stride;
  t.stride[1] = 1;
  return t;
}

static int fails = 0;
static uint64_t items_checked = 0;

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

// The position row that the stitching assigns to element i (< rd/2) of cos/sin, from the
// definitions: sections (cacheMode 0) or the interleaved rule (cacheMode 1).
static int assigned_row(const std::vector<int64_t> &sec, int64_t cache_mode, int64_t i) {
  if (sec.empty() || sec[0] == 0) return 0;
  if (cache_mode == 1) {
    if (i % 3 == 1 && i < 3 * sec[1]) return 1;
    if (i % 3 == 2 && i < 3 * sec[1]) return 2;
    return 0;
  }
  int64_t acc = 0;
  for (size_t k = 0; k < sec.size(); ++k) {
    acc += sec[k];
    if (i < acc) return int(k);
  }
  return -1;
}

// The wavefront kernel's position row for element j of the chunk starting at cos element i0
// (3-section plans on the multi-row path), as the kernel computes it, without branches.
static int wave_multi_row(const CachePlan &p, uint32_t i0, int j) {
  const uint32_t e = i0 + uint32_t(j);
  uint32_t m = i0 % 3u + uint32_t(j % 3);
  m = m >= 3u ? m - 3u : m;
  const int ri = int32_t(e) < p.interleave_end ? int(m) : 0;
  const int rs = int(int32_t(e) >= p.sec_end[0]) + int(int32_t(e) >= p.sec_end[1]);
  return p.interleaved ? ri : rs;
}

// The wavefront path (plan.wave): waves of 64 lanes, wave gw -> token gw / wave_wpt and head
// group gw % wave_wpt; lane l -> unit l % units of head row l / units (idle from wave_hpw up);
// wave_rows head rows of wave_hpw heads.  Checks that every output element is written
// once from its own input element, that every load (idle and clamped lanes included) stays
// inside the input rows, that a rotated element reads the cos|sin entry of its own pair, and
// that the position row of each cos|sin element is the one the stitching assigns.
static bool walk_waves(const CachePlan &p, bool neox, int64_t T, int64_t nq, int64_t nk,
                       int64_t H, int64_t rd, const std::vector<int64_t> &sec,
                       int64_t cache_mode, int64_t qs) {
  const int64_t V = p.vec, half = rd / 2, nh = nq + nk;
  const int64_t C = neox ? V : V / 2;
  const uint32_t lanes = p.wave_lin ? 2 * p.units : p.units;  // lanes per head
  CHECK(!p.wave_lin || (neox && !p.wave_xch), "one-vector NeoX units on a GPT-J or exchange plan");
  CHECK(lanes >= 1 && lanes <= 64 && p.wave_hpw == 64 / lanes, "wave plan lanes %u hpw %u",
        lanes, p.wave_hpw);
  const bool pair_units = neox && !p.wave_xch && !p.wave_lin && !p.multi_row;
  CHECK(p.wave_rows == (pair_units ? kWaveRowsPairUnits : kWaveRowsVectorUnits),
        "wave rows %u", p.wave_rows);
  CHECK(p.wave_heads == p.wave_rows * p.wave_hpw, "wave heads %u", p.wave_heads);
  CHECK(p.wave_block == uint32_t(neox ? kWaveBlockNeox : kWaveBlockGptj) && p.wave_block % 64 == 0,
        "wave workgroup of %u lanes", p.wave_block);
  // the scalar cos|sin row: GPT-J rope mode, a 128-byte row (two 64-byte scalar loads, eight
  // 8-byte chunks per half), launches of at least kScalarRowMinWaves wavefronts
  const int64_t esz = 16 / V;
  CHECK(p.wave_scalar_row == (!neox && sec.empty() && rd * esz == kScalarRowBytes &&
                              p.waves >= kScalarRowMinWaves),
        "scalar row %d for neox=%d rd %lld waves %lld", int(p.wave_scalar_row), int(neox),
        (long long)rd, (long long)p.waves);
  CHECK(!p.wave_scalar_row || (C * esz == 8 && half / C == 8), "scalar-row chunks");
  CHECK(int64_t(p.wave_wpt) * p.wave_heads >= nh &&
            int64_t(p.wave_wpt - 1) * p.wave_heads < nh, "waves per token %u", p.wave_wpt);
  CHECK(p.waves == T * int64_t(p.wave_wpt) && p.waves < kMaxWaves, "waves %lld",
        (long long)p.waves);
  std::vector<uint8_t> hq(size_t(T * nq * H), 0), hk(size_t(T * nk * H), 0);
  for (int64_t gw = 0; gw < p.waves; ++gw) {
    const uint32_t t32 = fastdiv_host(p.div_wpt, uint32_t(gw));
    CHECK(t32 == uint32_t(gw / p.wave_wpt), "wave %lld decodes to token %u", (long long)gw, t32);
    const int64_t t = t32;
    const int64_t hbase0 = int64_t(uint32_t(gw) - t32 * p.wave_wpt) * p.wave_heads;
    const bool xch = p.wave_xch, lin = p.wave_lin, exch = xch || lin;
    const uint32_t R = p.rot_units;
    for (uint32_t lane = 0; lane < 64; ++lane) {
      const uint32_t hsub = lane / lanes, u = lane - hsub * lanes;
      const bool on = hsub < p.wave_hpw;
      const int64_t hbase = hbase0 + (on ? hsub : 0);
      const bool rot = exch ? u < 2 * R : u < R;
      const uint32_t cu = !rot ? 0 : (exch && u >= R) ? u - R : u;
      const int64_t i0 = int64_t(cu) * C;
      if (exch && rot && on) {
        // the partner lane: same head row, unit u + R or u - R, whose first vector holds the
        // pair partners (column +- rd/2) of this lane's first vector
        const uint32_t pu = u < R ? u + R : u - R;
        const uint32_t pl = lane - u + pu;
        CHECK(pl < 64 && pl / lanes == hsub && pu < 2 * R, "lane %u partner lane %u", lane, pl);
        const int64_t mine = int64_t(u) * V, theirs = int64_t(pu) * V;
        CHECK(theirs - mine == (u < R ? half : -half), "lane %u partner at %lld, own %lld", lane,
              (long long)theirs, (long long)mine);
      }
      CHECK(i0 + C <= half, "cos chunk [%lld, %lld) beyond rd/2", (long long)i0,
            (long long)(i0 + C));
      // rows of the chunk's elements: one row (the section of i0) unless multi-row
      int first = -1;
      for (int64_t j = 0; j < C; ++j) {
        const int want = assigned_row(sec, cache_mode, i0 + j);
        int got;
        if (p.multi_row) {
          got = wave_multi_row(p, uint32_t(i0), int(j));
        } else if (p.mrope) {
          got = int(i0 >= p.sec_end[0]) + int(i0 >= p.sec_end[1]) +
                (p.nsec == 4 ? int(i0 >= p.sec_end[2]) : 0);
        } else {
          got = 0;
        }
        if (first < 0) first = got;
        CHECK(got == want, "lane %u element %lld: row %d, stitching assigns %d", lane,
              (long long)(i0 + j), got, want);
        CHECK(got < (p.mrope ? p.nsec : 1), "row %d beyond the position rows", got);
      }
      std::vector<int64_t> offs;
      if (xch) {
        CHECK(neox && 2 * rd <= H, "exchange layout on a plan with rd %lld, H %lld",
              (long long)rd, (long long)H);
        offs = {int64_t(u) * V, H / 2 + int64_t(u) * V};
      } else if (lin) {
        offs = {int64_t(u) * V};
      } else if (neox) {
        if (rot) {
          offs = {int64_t(u) * V, half + int64_t(u) * V};
        } else {
          const int64_t w = int64_t(u - R) * V;
          offs = {rd + w, rd + (H - rd) / 2 + w};
        }
      } else {
        offs = {int64_t(u) * V};
      }
      for (int k = 0; k < int(p.wave_rows); ++k) {
        const int64_t h = hbase + int64_t(k) * p.wave_hpw;
        const int64_t hl = h < nh ? h : nh - 1;  // the head the loads address
        const bool lq = hl < nq;
        const int64_t lrow = t * (lq ? qs : nk * H) + (lq ? hl : hl - nq) * H;
        for (int64_t o : offs)
          CHECK(o >= 0 && o + V <= H && lrow + o + V <= T * (lq ? qs : nk * H),
                "load outside the input rows");
        if (!on || h >= nh) continue;
        const bool is_q = h < nq;
        // stores address the token's q (or k) output row as one buffer range, in bytes
        const int64_t row_len = (is_q ? nq : nk) * H, es = 16 / V;
        CHECK(row_len * es < (int64_t(1) << 31), "output row of %lld bytes on the wave path",
              (long long)(row_len * es));
        const int64_t in_row = (is_q ? h : h - nq) * H;
        const int64_t out_row = t * row_len + in_row;
        std::vector<uint8_t> &hit = is_q ? hq : hk;
        for (size_t a = 0; a < offs.size(); ++a)
          for (int64_t e = 0; e < V; ++e) {
            const int64_t col = offs[a] + e;
            // the exchange layout rotates only the first access of a rotated lane
            const bool rotated = exch ? (rot && a == 0) : rot;
            CHECK(rotated == (col < rd), "column %lld on the wrong side of rotaryDim",
                  (long long)col);
            CHECK(in_row + col >= 0 && in_row + col < row_len,
                  "store outside the token's output row");
            const size_t oi = size_t(out_row + col);
            CHECK(hit[oi] == 0, "wave output %zu written twice", oi);
            hit[oi] = 1;
            if (rotated) {
              const int64_t pair = neox ? (col < half ? col : col - half) : col / 2;
              const int64_t cs = i0 + (neox ? e : e / 2);
              CHECK(pair == cs, "column %lld reads cos %lld, wants %lld", (long long)col,
                    (long long)cs, (long long)pair);
            }
          }
        ++items_checked;
      }
    }
  }
  for (size_t i = 0; i < hq.size(); ++i) CHECK(hq[i] == 1, "wave q output %zu unwritten", i);
  for (size_t i = 0; i < hk.size(); ++i) CHECK(hk[i] == 1, "wave k output %zu unwritten", i);
  return true;
}

static int wave_plans = 0, xch_plans = 0, lin_plans = 0, pair_plans = 0, wide_pair_plans = 0,
           scalar_row_plans = 0;
// Every g_stride-th plan is walked (1: all of them); runs under the sanitizers use a sparser
// sample of the same plans.
static int g_stride = 1, g_seen = 0, g_walked = 0;

static bool walk(rope_dtype dt, bool neox, int64_t T, int64_t nq, int64_t nk, int64_t H,
                 int64_t rd, std::vector<int64_t> sec, int64_t cache_mode, int64_t q_pad,
                 uintptr_t pos_offset = 0) {
  if (g_seen++ % g_stride != 0) return true;
  ++g_walked;
  const int64_t m = sec.empty() ? 0 : int64_t(sec.size());
  rope_tensor pos{};
  pos.data = reinterpret_cast<void *>(uintptr_t(0x20000000) + pos_offset);
  pos.dtype = ROPE_I64;
  if (m) {
    pos.ndim = 2;
    pos.shape[0] = m;
    pos.shape[1] = T;
    pos.stride[0] = T;
    pos.stride[1] = 1;
  } else {
    pos.ndim = 1;
    pos.shape[0] = T;
    pos.stride[0] = 1;
  }
  const int64_t qs = nq * H + q_pad;
  const rope_tensor q = t2(0x30000000, dt, T, nq * H, qs);
  const rope_tensor k = t2(0x50000000, dt, T, nk * H, nk * H);
  const rope_tensor c = t2(0x70000000, dt, 1024, rd, rd);  // below 0x80000000 up to rd 65536
  const rope_tensor qo = t2(0x80000000, dt, T, nq * H, nq * H);
  const rope_tensor ko = t2(0xA0000000, dt, T, nk * H, nk * H);
  CachePlan p;
  std::string err;
  const int st = plan_cache(&pos, &q, &k, &c, m ? sec.data() : nullptr, m, H, neox ? 1 : 0,
                            cache_mode, &qo, &ko, &p, &err);
  CHECK(st == ROPE_OK, "plan rejected: %s", err.c_str());
  CHECK(T > 256 * 7 || p.tile_tokens == 1, "%lld tokens fit one round of workgroups but "
        "share tiles of %u", (long long)T, p.tile_tokens);
  const int64_t V = p.vec, half = rd / 2;
  const int64_t es = dt == ROPE_F32 ? 4 : 2;
  CHECK(V * es == 16, "vector of %lld elements", (long long)V);
  const int64_t lds_elems = int64_t(p.tile_tokens) * rd;  // the LDS the launch requests
  std::vector<uint8_t> hq(size_t(T * nq * H), 0), hk(size_t(T * nk * H), 0);
  std::vector<uint8_t> tok_seen(size_t(T), 0);
  for (int64_t tile = 0; tile < p.tiles; ++tile) {
    int64_t t0, ntok;  // the kernel's tile -> tokens map (tapered end: one-token tiles)
    if (tile < p.big_tiles) {
      t0 = tile * int64_t(p.tile_tokens);
      ntok = int64_t(p.tile_tokens);
    } else {
      t0 = p.big_tokens + (tile - p.big_tiles);
      ntok = 1;
    }
    CHECK(ntok >= 1 && t0 >= 0 && t0 + ntok <= T, "tile %lld covers tokens [%lld, %lld)",
          (long long)tile, (long long)t0, (long long)(t0 + ntok));
    for (int64_t t = t0; t < t0 + ntok; ++t) {
      CHECK(tok_seen[size_t(t)] == 0, "token %lld in two tiles", (long long)t);
      tok_seen[size_t(t)] = 1;
    }
    // direct plans (rope mode, a cos|sin row of more than 16384 elements): nothing is staged,
    // each item reads its pair indices from the cache row (checked with the items below)
    CHECK(p.cs_direct == (rd > 16384), "direct cos/sin reads %d for rotaryDim %lld",
          int(p.cs_direct), (long long)rd);
    CHECK(!p.cs_direct || (m == 0 && p.tile_tokens == 1 && !p.wave),
          "direct plan with %lld position rows, %u-token tiles", (long long)m, p.tile_tokens);
    // staging: one lane per chunk, or for multi-row plans (16-byte cache rows) one lane per
    // (chunk, row of rows 0..2) writing only the elements assigned to its row
    std::vector<uint8_t> lds(size_t(p.cs_direct ? 0 : lds_elems), 0);
    const uint32_t stage_items = p.cs_direct ? 0u : uint32_t(ntok) * p.stage_chunks;
    const bool per_row = p.multi_row && p.cache_vec;
    CHECK(!p.multi_row || m == 3, "multi-row plan with %lld position rows", (long long)m);
    for (uint32_t idx = 0; idx < stage_items * (per_row ? 3u : 1u); ++idx) {
      const uint32_t chunk = per_row ? idx / 3u : idx;
      const int lane_row = per_row ? int(idx % 3u) : -1;
      const uint32_t tl = fastdiv_host(p.div_stage, chunk);
      const int64_t i0 = int64_t(chunk - tl * p.stage_chunks) * V;
      CHECK(tl < uint32_t(ntok) && i0 + V <= half, "staging chunk %u", chunk);
      int first_row = assigned_row(sec, cache_mode, i0);
      for (int64_t e = 0; e < V; ++e) {
        const int r = assigned_row(sec, cache_mode, i0 + e);
        CHECK(r >= 0 && (m == 0 ? r == 0 : r < m), "row %d", r);
        CHECK(p.multi_row || r == first_row,
              "chunk at %lld mixes rows %d and %d without the multi-row path", (long long)i0,
              first_row, r);
        if (per_row && r != lane_row) continue;
        for (int64_t h2 : {int64_t(0), half}) {
          const int64_t li = int64_t(tl) * rd + h2 + i0 + e;
          CHECK(li < lds_elems, "LDS index %lld beyond %lld", (long long)li,
                (long long)lds_elems);
          CHECK(lds[size_t(li)] == 0, "LDS element %lld staged twice", (long long)li);
          lds[size_t(li)] = 1;
        }
      }
    }
    for (int64_t i = 0; !p.cs_direct && i < ntok * rd; ++i)
      CHECK(lds[size_t(i)] == 1, "LDS %lld unset", (long long)i);
    // items
    const uint32_t tile_items = uint32_t(ntok) * p.items_per_token;
    for (uint32_t it = 0; it < tile_items; ++it) {
      const uint32_t tl = fastdiv_host(p.div_ipt, it);
      const uint32_t r = it - tl * p.items_per_token;
      const uint32_t h = fastdiv_host(p.div_units, r);
      const uint32_t u = r - h * p.units;
      CHECK(tl < uint32_t(ntok) && h < uint32_t(nq + nk), "item %u", it);
      const int64_t t = t0 + tl;
      const bool is_q = h < uint32_t(nq);
      const int64_t hh = is_q ? int64_t(h) : int64_t(h) - nq;
      const int64_t in_row = t * (is_q ? qs : nk * H) + hh * H;
      const int64_t out_row = t * ((is_q ? nq : nk) * H) + hh * H;
      std::vector<uint8_t> &hit = is_q ? hq : hk;
      std::vector<int64_t> offs;
      const bool rotated = u < p.rot_units;
      if (neox) {
        if (rotated) {
          offs = {int64_t(u) * V, half + int64_t(u) * V};
        } else {
          const int64_t v = int64_t(u - p.rot_units) * V;
          offs = {rd + v, rd + (H - rd) / 2 + v};
        }
      } else {
        offs = {int64_t(u) * V};
      }
      for (size_t a = 0; a < offs.size(); ++a)
        for (int64_t e = 0; e < V; ++e) {
          const int64_t col = offs[a] + e;  // position inside the head
          CHECK(col >= 0 && col < H, "column %lld outside the head", (long long)col);
          CHECK(rotated == (col < rd), "column %lld on the wrong side of rotaryDim",
                (long long)col);
          CHECK(in_row + col < T * qs || !is_q, "q input out of bounds");
          const size_t oi = size_t(out_row + col);
          CHECK(hit[oi] == 0, "output %zu written twice", oi);
          hit[oi] = 1;
          if (rotated) {
            // the pair index whose cos|sin this element uses
            const int64_t pair = neox ? (col < half ? col : col - half) : col / 2;
            const int64_t lds_cos = neox ? int64_t(u) * V + e : int64_t(u) * (V / 2) + e / 2;
            CHECK(pair == lds_cos, "column %lld reads cos %lld, wants %lld", (long long)col,
                  (long long)lds_cos, (long long)pair);
            if (neox && a == 1)
              CHECK(offs[1] - offs[0] == half, "NeoX halves not rd/2 apart");
          }
        }
      ++items_checked;
    }
  }
  for (size_t t = 0; t < tok_seen.size(); ++t) CHECK(tok_seen[t] == 1, "token %zu in no tile", t);
  for (size_t i = 0; i < hq.size(); ++i) CHECK(hq[i] == 1, "q output %zu unwritten", i);
  for (size_t i = 0; i < hk.size(); ++i) CHECK(hk[i] == 1, "k output %zu unwritten", i);
  // the wavefront path: taken exactly when its conditions hold (16-byte access everywhere,
  // at most 64 units per head, aligned positions); then walked as the kernel walks it
  const uint32_t lanes = p.wave_lin ? 2 * p.units : p.units;
  const int64_t row_limit = int64_t(1) << 31;
  const bool wave_ok = p.vector_io && p.cache_vec && lanes <= 64 && pos_offset % 8 == 0 &&
                       nq * H * es < row_limit && nk * H * es < row_limit;
  CHECK(p.wave == wave_ok, "wave path %d, conditions say %d", int(p.wave), int(wave_ok));
  // the NeoX layout is a speed choice; each is walked below, and the exchange layout needs
  // rd <= H/2 (all rotated vectors in the first access)
  CHECK(!p.wave_xch || (wave_ok && neox && !p.wave_lin && 2 * rd <= H),
        "exchange layout %d for neox=%d rd %lld H %lld", int(p.wave_xch), int(neox),
        (long long)rd, (long long)H);
  if (p.wave) {
    ++wave_plans;
    xch_plans += p.wave_xch ? 1 : 0;
    lin_plans += p.wave_lin ? 1 : 0;
    pair_plans += neox && !p.wave_xch && !p.wave_lin ? 1 : 0;
    wide_pair_plans += neox && !p.wave_xch && !p.wave_lin && p.units > 32 ? 1 : 0;
    scalar_row_plans += p.wave_scalar_row ? 1 : 0;
    return walk_waves(p, neox, T, nq, nk, H, rd, sec, cache_mode, qs);
  }
  return true;
}

// Plan only (no walk): whether a one-token rope-mode plan with nq + nk heads of H elements
// takes the wavefront path.  Tensors sit 2^40 bytes apart, so that rows of several GiB overlap
// nothing.
static int wave_taken(rope_dtype dt, int64_t nq, int64_t nk, int64_t H) {
  rope_tensor pos{};
  pos.data = reinterpret_cast<void *>(uintptr_t(6) << 40);
  pos.dtype = ROPE_I64;
  pos.ndim = 1;
  pos.shape[0] = 1;
  pos.stride[0] = 1;
  const rope_tensor q = t2(uintptr_t(1) << 40, dt, 1, nq * H, nq * H);
  const rope_tensor k = t2(uintptr_t(2) << 40, dt, 1, nk * H, nk * H);
  const rope_tensor c = t2(uintptr_t(5) << 40, dt, 1024, H, H);
  const rope_tensor qo = t2(uintptr_t(3) << 40, dt, 1, nq * H, nq * H);
  const rope_tensor ko = t2(uintptr_t(4) << 40, dt, 1, nk * H, nk * H);
  CachePlan p;
  std::string err;
  const int st = plan_cache(&pos, &q, &k, &c, nullptr, 0, H, 1, 0, &qo, &ko, &p, &err);
  if (st != ROPE_OK) {
    std::printf("FAIL: plan rejected: %s\n", err.c_str());
    return -1;
  }
  return p.wave ? 1 : 0;
}

int main(int argc, char **argv) {
  if (argc > 1 && std::atoi(argv[1]) > 1) g_stride = std::atoi(argv[1]);
  int plans = 0;
  const std::vector<std::vector<int64_t>> mlists = {
      {}, {16, 24, 24}, {8, 12, 12}, {24, 20, 20}, {11, 11, 10}, {16, 16, 16, 16}};
  for (rope_dtype dt : {ROPE_F32, ROPE_F16, ROPE_BF16}) {
    const int64_t align = 64 / (dt == ROPE_F32 ? 4 : 2);
    for (bool neox : {true, false})
      for (const auto &sec : mlists)
        for (int64_t cm : {int64_t(0), int64_t(1)}) {
          if (cm == 1 && sec.size() != 3) continue;
          std::vector<int64_t> rds;
          if (sec.empty()) rds = {align, 2 * align, 4 * align};
          else rds = {2 * (sec[0] + sec[1] + sec[2] + (sec.size() == 4 ? sec[3] : 0))};
          for (int64_t rd : rds)
            for (int64_t extra : {int64_t(0), align, 2 * align})
              for (int64_t T : {int64_t(1), int64_t(7), int64_t(61), int64_t(1792),
                                int64_t(1793), int64_t(5123)})
                for (auto hq : {std::pair<int64_t, int64_t>{1, 1}, {5, 3}, {32, 8}}) {
                  if (T > 1000 && hq.first != 1) continue;  // the long case: one head each
                  const int64_t pad = (T == 7) ? align : 0;
                  if (!walk(dt, neox, T, hq.first, hq.second, rd + extra, rd, sec, cm, pad))
                    return 1;
                  ++plans;
                }
        }
  }
  // wide NeoX heads on the wavefront path: 20 to 64 units (lanes) a head, rotaryDim H and H/2
  // (units a multiple of 4, so that H/2 is a 64-byte multiple)
  for (rope_dtype dt : {ROPE_F32, ROPE_BF16}) {
    const int64_t v = dt == ROPE_F32 ? 4 : 8;
    for (int64_t units : {int64_t(20), int64_t(32), int64_t(36), int64_t(48), int64_t(64)})
      for (int64_t T : {int64_t(1), int64_t(9), int64_t(300)}) {
        const int64_t H = 2 * v * units;
        if (!walk(dt, true, T, 3, 2, H, H, {}, 0, 0)) return 1;
        if (!walk(dt, true, T, 2, 1, H, H / 2, {}, 0, 0)) return 1;
        plans += 2;
      }
  }
  // plans the wavefront path does not take: heads of more than 64 units, positions not
  // 8-byte aligned
  for (rope_dtype dt : {ROPE_F32, ROPE_BF16})
    for (bool neox : {true, false}) {
      const int64_t v = dt == ROPE_F32 ? 4 : 8;
      const int64_t H = (neox ? 2 : 1) * v * 72;  // 72 units per head
      for (int64_t T : {int64_t(1), int64_t(9)}) {
        if (!walk(dt, neox, T, 3, 2, H, H / 2, {}, 0, 0)) return 1;
        if (!walk(dt, neox, T, 2, 1, H, H, {}, 0, 0, 4)) return 1;
        plans += 2;
      }
      if (!walk(dt, neox, 5, 3, 1, 128, 128, {16, 24, 24}, 0, 0, 2)) return 1;
      ++plans;
      // rotaryDim at the LDS tile's limit (16384) and past it (direct cos/sin reads)
      const int64_t align = dt == ROPE_F32 ? 16 : 32;
      for (int64_t rd : {int64_t(16384), 16384 + align, int64_t(24576)})
        for (int64_t extra : {int64_t(0), align}) {
          if (!walk(dt, neox, 3, 2, 1, rd + extra, rd, {}, 0, 0)) return 1;
          ++plans;
        }
    }
  // the wavefront kernel stores through one buffer range per token's q (or k) output row, of
  // 32-bit offsets: a row of 2^31 bytes or more goes to the tile form (bf16 heads of 256 B)
  for (int64_t nk : {int64_t(1), (int64_t(1) << 23) - 1, int64_t(1) << 23}) {
    const int64_t nq = nk == 1 ? (int64_t(1) << 23) : 1;
    const int want = (nq < (int64_t(1) << 23) && nk < (int64_t(1) << 23)) ? 1 : 0;
    const int got = wave_taken(ROPE_BF16, nq, nk, 128);
    if (got != want) {
      std::printf("FAIL: nq %lld nk %lld heads of 256 B: wavefront path %d, want %d\n",
                  (long long)nq, (long long)nk, got, want);
      return 1;
    }
    ++plans;
  }
  if (wave_plans == 0 || wave_plans == g_walked || xch_plans == 0 || lin_plans == 0 ||
      pair_plans == 0 || wide_pair_plans == 0 || (scalar_row_plans == 0 && g_stride == 1)) {
    std::printf("FAIL: %d of %d plans take the wavefront path (%d exchange, %d one-vector "
                "NeoX, %d pair units, %d of them over 32 lanes a head, %d scalar-row GPT-J); "
                "every path and layout must be covered\n",
                wave_plans, g_walked, xch_plans, lin_plans, pair_plans, wide_pair_plans,
                scalar_row_plans);
    return 1;
  }
  std::printf("ok %d %llu (%d walked, %d on the wavefront path: %d exchange, %d one-vector "
              "NeoX, %d pair units, %d of them over 32 lanes a head, %d scalar-row GPT-J)\n",
              plans, (unsigned long long)items_checked, g_walked, wave_plans, xch_plans,
              lin_plans, pair_plans, wide_pair_plans, scalar_row_plans);
  return 0;
}
