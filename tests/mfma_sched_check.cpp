// CPU check of the MFMA consumer's integer schedule (mfma_sched.h), the same
// functions the kernel runs. It replays, per workgroup, the kernel's compute
// walk and its direct-load cursor (prologue of STAGES-1 steps, then one
// cursor step per k-step, the cursor running STAGES-1 steps ahead and
// re-loading the last step once the work is out), and checks:
//   - every k-step of every output tile is computed by exactly one workgroup
//     and, with the split, the tile's contributors are consecutive runs in
//     shard order with distinct partial slots below 2G;
//   - the cursor loads exactly the step the compute walk consumes from that
//     buffer: right tile, right shard buffer, right column and B rows;
//   - every 16-byte lane load lies inside its shard buffer (inbox or source
//     shards, and the BSP gather buffer; row-major and in 32-column k-panels)
//     and inside B, reads the element it stands for, and a stage's chunks
//     cover each (row, chunk) of the tile exactly once (swizzle bijective);
//   - gated launches: a flag tile is gated before any load from it, under
//     three models of what a flag poll reveals (only the awaited tile, all,
//     random subsets), and tracking stops only once every flag is seen;
//   - arrival order: every k-step of a tile is loaded exactly once, each
//     chosen flag tile is real (< T) and untaken, from the same loads.
// Exit status 0 when every check passes; the first failure is printed.
// Built with -DPLANT=1 (a flag-tile crossing skips its gate) or -DPLANT=2 (a
// shard crossing keeps the old column offset), the replay carries a planted
// mistake that the checks must catch.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <set>
#include <vector>

#include "mfma_sched.h"

#ifndef PLANT
#define PLANT 0
#endif

using namespace agemm::sched;

namespace {

struct Cfg {
  int BM, BN, BK, STAGES;
};

struct Shape {
  int64_t M, N;
  int W, KS, BKf;
  Cfg cfg;
  int G;
  bool split;
};

long long g_checks = 0;
char g_fail[512];

#define CHECK(cond, ...)                                                        \
  do {                                                                          \
    ++g_checks;                                                                 \
    if (!(cond)) {                                                              \
      std::snprintf(g_fail, sizeof g_fail, __VA_ARGS__);                        \
      return false;                                                             \
    }                                                                           \
  } while (0)

struct Load {
  int w, ct;       // tile and k-step the cursor stands on
  int shard;       // A buffer the loads use
  int64_t a_col;   // column (elements) inside the shard of the k-step's first column
  int64_t b_row;   // first B row of the k-step
};

// Lane loads of one cursor step in bounds; chunks cover the tile once.
bool check_lane_loads(const Shape& s, int w, const Load& L, const TileGrid& tg) {
  const Cfg& c = s.cfg;
  int mb, nb;
  tile_coords(tg, s.split, w, mb, nb);
  const int64_t m0 = (int64_t)mb * c.BM, n0 = (int64_t)nb * c.BN;
  const int rmax = (int)(s.M - 1 - m0);
  const int cmax = (int)(s.N - 8 - n0);
  const int64_t K = (int64_t)s.W * s.KS;
  // four A layouts: row-major shard buffers (lda = KS) and BSP gather buffer
  // (lda = K); the k-panel layout of the inbox and of the gather buffer
  // (32-column panels of M rows of 64 bytes, shard after shard)
  for (int layout = 0; layout < 4; ++layout) {
    const bool gathered = layout & 1, panels = layout >= 2;
    const int64_t lda = gathered ? K : s.KS;
    const int64_t base = !gathered ? 0 : panels ? (int64_t)L.shard * s.M * s.KS * 2 : (int64_t)L.shard * s.KS * 2;
    const int64_t buf_bytes = gathered ? s.M * K * 2 : s.M * s.KS * 2;
    const int64_t pb = s.M * 64;  // bytes of one panel
    const int cpr = c.BK / 8;
    std::vector<int> seen((size_t)c.BM * cpr, 0);
    for (int q = 0; q < c.BM * cpr; ++q) {
      uint32_t off;
      if (panels) off = c.BK == 32 ? a_src_offset_panels<32>(q, rmax, pb) : a_src_offset_panels<64>(q, rmax, pb);
      else off = c.BK == 32 ? a_src_offset<32>(q, rmax, lda * 2) : a_src_offset<64>(q, rmax, lda * 2);
      // the kernel's cursor: tile's first row, plus one k-step's bytes per step
      const int64_t cursor = panels ? base + m0 * 64 + (L.a_col / 32) * pb : base + m0 * lda * 2 + L.a_col * 2;
      const int64_t addr = cursor + off;
      CHECK(addr >= 0 && addr + 16 <= buf_bytes,
            "A load out of bounds: layout %d tile %d step %d q %d addr %lld size %lld", layout, w, L.ct, q,
            (long long)addr, (long long)buf_bytes);
      const int r = q / cpr;
      const int ch = (q % cpr) ^ (c.BK == 32 ? swz_a<4>(r) : swz_a<8>(r));
      CHECK(ch >= 0 && ch < cpr, "A swizzled chunk out of range");
      if (r <= rmax) {  // rows past M are clamped and never stored
        const int64_t col = L.a_col + ch * 8;  // element column inside the shard
        const int64_t want = panels ? base + ((col / 32) * s.M + m0 + r) * 64 + (col % 32) * 2
                                    : base + (m0 + r) * lda * 2 + col * 2;
        CHECK(addr == want, "A chunk %d of row %d at the wrong source (layout %d)", ch, r, layout);
        seen[(size_t)r * cpr + ch]++;
      }
    }
    for (int r = 0; r <= rmax && r < c.BM; ++r)
      for (int ch = 0; ch < cpr; ++ch)
        CHECK(seen[(size_t)r * cpr + ch] == 1, "A (row %d, chunk %d) loaded %d times", r, ch,
              seen[(size_t)r * cpr + ch]);
  }
  const int64_t b_bytes = K * s.N * 2;
  const int cprb = c.BN / 8;
  std::vector<int> seen((size_t)c.BK * cprb, 0);
  for (int q = 0; q < c.BK * cprb; ++q) {
    const uint32_t off = c.BN == 256 ? b_src_offset<256>(q, cmax, s.N) : b_src_offset<128>(q, cmax, s.N);
    const int64_t addr = n0 * 2 + L.b_row * s.N * 2 + off;
    CHECK(addr >= 0 && addr + 16 <= b_bytes, "B load out of bounds: tile %d step %d q %d", w, L.ct, q);
    const int k = q / cprb;
    const int col = ((q % cprb) ^ swz_b(k)) * 8;
    CHECK(col >= 0 && col < c.BN, "B swizzled chunk out of range");
    if (col <= cmax) {  // columns past N are clamped and never stored
      CHECK(addr == n0 * 2 + (L.b_row + k) * s.N * 2 + col * 2, "B chunk at the wrong source");
      seen[(size_t)k * cprb + col / 8]++;
    }
  }
  for (int k = 0; k < c.BK; ++k)
    for (int ch = 0; ch < cprb && ch * 8 <= cmax; ++ch)
      CHECK(seen[(size_t)k * cprb + ch] == 1, "B (k %d, chunk %d) loaded %d times", k, ch,
            seen[(size_t)k * cprb + ch]);
  return true;
}

// ready models: 0 = a poll reveals the awaited tile only, 1 = all, 2 = random subsets
struct Flags {
  int T, model;
  uint64_t ready, tmask;
  std::mt19937_64* rng;
  void poll(int tile) {
    if (model == 1) ready = tmask;
    else if (model == 2) ready |= ((*rng)() & tmask) | (1ull << tile);
    else ready |= 1ull << tile;
  }
};

bool run_shape(const Shape& s, int model, std::mt19937_64& rng, bool arrival) {
  const Cfg& c = s.cfg;
  const TileGrid tg = tile_grid(s.M, s.N, c.BM, c.BN, s.G);
  const int SPS = s.KS / c.BK;
  const int NS = s.W * SPS;
  const int KT = s.KS / s.BKf;
  const int spt = SPS / KT;
  const int T = s.W * KT;
  const uint64_t tmask = flag_mask(T);
  CHECK(s.G >= 1 && (s.split ? (int64_t)s.G <= (int64_t)tg.total * s.W : s.G <= tg.total), "bad grid");
  std::vector<int> done((size_t)tg.total * NS, 0);
  std::vector<std::vector<int>> contrib(tg.total);  // runs contributing to each tile
  for (int b = 0; b < s.G; ++b) {
    const Work wk = work_of(b, s.G, tg.total, s.W, SPS, s.split);
    // compute walk
    std::vector<std::pair<int, int>> comp;
    Seg ms;
    seg_first(wk, ms);
    do {
      CHECK(ms.w >= 0 && ms.w < tg.total && ms.kb >= 0 && ms.kb < ms.ke && ms.ke <= NS && ms.kb % SPS == 0 &&
                ms.ke % SPS == 0,
            "bad segment w=%d [%d,%d)", ms.w, ms.kb, ms.ke);
      if (s.split && (ms.kb != 0 || ms.ke != NS)) contrib[ms.w].push_back(wk.bp);
      for (int t = ms.kb; t < ms.ke; ++t) {
        comp.push_back({ms.w, t});
        done[(size_t)ms.w * NS + t]++;
      }
    } while (seg_next(wk, ms));

    // the load cursor, replayed as the kernel runs it
    Flags fl{T, model, 0, tmask, &rng};
    if (model == 2) fl.ready = rng() & tmask;  // the launch-time look at the flags
    std::vector<Load> loads;
    Seg cseg;
    seg_first(wk, cseg);
    KPos kp{};
    bool track = true;
    int a_shard = 0;
    int64_t a_col = 0, b_row = 0;  // emulated ca / cb
    // arrival state
    int act = 0, cfsub = 0;
    uint64_t taken = 0;
    auto gate = [&](int tile) -> bool {
      CHECK(tile >= 0 && tile < T, "gate of tile %d outside T=%d", tile, T);
      if (!((fl.ready >> tile) & 1)) fl.poll(tile);
      return true;
    };
    auto apply = [&](int f) -> bool {  // arrival: choice published and applied
      CHECK(f >= 0 && f < T && !((taken >> f) & 1), "arrival chose tile %d (T=%d, taken %llx)", f, T,
            (unsigned long long)taken);
      taken |= 1ull << f;
      const int step = flag_first_step(f, KT, SPS, spt);
      a_shard = f / KT;
      a_col = (int64_t)(step - a_shard * SPS) * c.BK;
      b_row = (int64_t)step * c.BK;
      return gate(f);
    };
    auto choose_apply = [&]() -> bool {
      if ((fl.ready & ~taken & tmask) == 0) fl.poll(arrival_pick(0, taken, tmask));
      return apply(arrival_pick(fl.ready, taken, tmask));
    };
    auto enter = [&]() -> bool {
      if (arrival) {
        act = 0;
        cfsub = 0;
        taken = 0;
        return choose_apply();
      }
      kpos_enter(kp, cseg, SPS, spt, KT, track);
      a_shard = kp.cs;
      a_col = 0;
      b_row = (int64_t)cseg.kb * c.BK;
      CHECK(kp.cft == a_shard * KT, "flag tile at entry");
      return gate(kp.cft);
    };
    auto advance = [&]() -> bool {
      if (arrival) {
        if (++act == cseg.ke) {
          if (seg_next(wk, cseg)) return enter();
          act = cseg.ke - 1;
          return true;
        }
        if (++cfsub == spt) {
          cfsub = 0;
          return choose_apply();
        }
        a_col += c.BK;
        b_row += c.BK;
        return true;
      }
      a_col += c.BK;
      b_row += c.BK;
      if (!kpos_step(kp, cseg.ke)) return true;
      if (kp.ct == cseg.ke) {
        if (seg_next(wk, cseg)) return enter();
        a_col -= c.BK;
        b_row -= c.BK;
        kp.ct = cseg.ke - 1;
        return true;
      }
      const int ev = kpos_event(kp, cseg.ke, SPS, spt, track);
      if (ev & kEvShard) {
        a_shard = kp.cs;
#if PLANT != 2
        a_col = 0;
#endif
      }
      if (ev & kEvFlag) {
#if PLANT != 1
        if (!gate(kp.cft)) return false;
#endif
        if ((fl.ready & tmask) == tmask) track = false;
      }
      return true;
    };
    auto record = [&]() -> bool {
      const int ct = arrival ? -1 : kp.ct;
      loads.push_back({cseg.w, ct, a_shard, a_col, b_row});
      // the flag tile of the loaded step must have been seen raised
      const int f = a_shard * KT + (int)(a_col / c.BK) / spt;
      CHECK((fl.ready >> f) & 1, "load of flag tile %d before its gate (tile %d)", f, cseg.w);
      // lane offsets depend on the tile only: check them at the first and last
      // k-step of each shard (the extremes of the column offset)
      if (a_col == 0 || a_col == (int64_t)(SPS - 1) * c.BK) return check_lane_loads(s, cseg.w, loads.back(), tg);
      return true;
    };
    if (!enter()) return false;
    const size_t steps = comp.size() + (size_t)(c.STAGES - 1);
    for (size_t i = 0; i < steps; ++i) {
      if (!record()) return false;
      if (!advance()) return false;
    }
    // compare the loads with the compute walk
    for (size_t i = 0; i < comp.size(); ++i) {
      const Load& L = loads[i];
      CHECK(L.w == comp[i].first, "load %zu of tile %d, compute tile %d", i, L.w, comp[i].first);
      if (!arrival) {
        const int t = comp[i].second;
        CHECK(L.ct == t && L.shard == t / SPS && L.a_col == (int64_t)(t % SPS) * c.BK && L.b_row == (int64_t)t * c.BK,
              "load %zu: step %d shard %d col %lld row %lld, compute step %d", i, L.ct, L.shard, (long long)L.a_col,
              (long long)L.b_row, t);
      }
    }
    if (arrival) {
      // per tile: the k-steps loaded are exactly 0..NS-1 once each
      size_t i = 0;
      while (i < comp.size()) {
        const int w = comp[i].first;
        std::vector<int> cnt(NS, 0);
        size_t j = i;
        for (; j < comp.size() && comp[j].first == w && j - i < (size_t)NS; ++j) {
          const Load& L = loads[j];
          CHECK(L.w == w, "arrival load of another tile");
          const int64_t step = L.shard * (int64_t)SPS + L.a_col / c.BK;
          CHECK(L.b_row == step * c.BK && step >= 0 && step < NS, "arrival A/B steps differ");
          cnt[(size_t)step]++;
        }
        for (int t = 0; t < NS; ++t) CHECK(cnt[t] == 1, "arrival: tile %d step %d loaded %d times", w, t, cnt[t]);
        i = j;
      }
    }
    // the extra cursor steps re-load the last step
    for (size_t i = comp.size(); i < loads.size(); ++i) {
      const Load& a = loads[i];
      const Load& z = loads[comp.size() - 1];
      CHECK(a.w == z.w && a.shard == z.shard && a.a_col == z.a_col && a.b_row == z.b_row, "tail re-load differs");
    }
  }
  for (int w = 0; w < tg.total; ++w)
    for (int t = 0; t < NS; ++t)
      CHECK(done[(size_t)w * NS + t] == 1, "tile %d step %d computed %d times", w, t, done[(size_t)w * NS + t]);
  if (s.split) {
    for (int w = 0; w < tg.total; ++w) {
      const Work wk = work_of(0, s.G, tg.total, s.W, SPS, true);
      const int first = owner(wk, (int64_t)w * s.W);
      const int n = owner(wk, (int64_t)w * s.W + s.W - 1) - first + 1;
      const auto& v = contrib[w];
      if (v.empty()) {
        CHECK(n == 1, "tile %d whole but %d owners", w, n);
        continue;
      }
      CHECK((int)v.size() == n, "tile %d: %zu contributors, owners say %d", w, v.size(), n);
      std::set<int> slots;
      for (int j = 0; j < n; ++j) {
        CHECK(std::find(v.begin(), v.end(), first + j) != v.end(), "tile %d: run %d missing", w, first + j);
        const int sl = slot_of(wk, first + j, w);
        CHECK(sl >= 0 && sl < 2 * s.G && slots.insert(sl).second, "tile %d: slot %d repeated or out of range", w, sl);
      }
    }
  }
  return true;
}

}  // namespace

int main(int argc, char** argv) {
  const int budget = argc > 1 ? std::atoi(argv[1]) : 3000;
  std::mt19937_64 rng(0x5c4ed);
  const Cfg cfgs[] = {{256, 256, 32, 4}, {128, 128, 64, 4}, {256, 128, 32, 4}};
  const int Ws[] = {1, 2, 3, 4, 8, 16};
  int shapes = 0;
  // the benchmark workloads' launches (at small K so that the replay is quick)
  std::vector<Shape> list;
  list.push_back({4096, 28672, 8, 128, 128, cfgs[0], 256, false});
  list.push_back({512, 28672, 8, 128, 128, cfgs[0], 224, false});
  list.push_back({128, 28672, 8, 128, 128, cfgs[1], 224, false});
  list.push_back({256, 28672, 8, 128, 128, cfgs[0], 256, true});
  list.push_back({256, 28672, 8, 128, 128, cfgs[2], 224, false});
  list.push_back({192, 28672, 8, 128, 128, cfgs[2], 224, false});
  // the accepted size limits (32-bit lane offsets): N = 2^24 with one shard of
  // 64 columns (131,072 one-k-step tiles), K = 2^22 with W = 8 (split and whole)
  list.push_back({2, 1 << 24, 1, 64, 64, cfgs[1], 256, false});
  list.push_back({3, 136, 8, 1 << 19, 1 << 16, cfgs[1], 16, true});
  list.push_back({3, 136, 8, 1 << 19, 1 << 16, cfgs[0], 1, false});
  while ((int)list.size() < budget) {
    Shape s;
    s.cfg = cfgs[rng() % 3];
    s.W = Ws[rng() % 6];
    const int ks_units = 1 + (int)(rng() % 8);  // KS in 64s
    s.KS = 64 * ks_units;
    if (s.KS % s.cfg.BK) continue;
    // BKf: a multiple of 64 dividing KS with T <= 64
    std::vector<int> opts;
    for (int b = 64; b <= s.KS; b += 64)
      if (s.KS % b == 0 && (s.KS / b) * s.W <= 64 && b % s.cfg.BK == 0) opts.push_back(b);
    if (opts.empty()) continue;
    s.BKf = opts[rng() % opts.size()];
    s.M = 1 + (int64_t)(rng() % 1100);
    s.N = 8 * (1 + (int64_t)(rng() % 420));
    const TileGrid tg = tile_grid(s.M, s.N, s.cfg.BM, s.cfg.BN, 1);
    s.split = s.W >= 2 && (rng() % 3 == 0);
    const int64_t cap = s.split ? (int64_t)tg.total * s.W : tg.total;
    const int cus = 1 + (int)(rng() % 300);
    s.G = (int)(cap < cus ? cap : cus);
    list.push_back(s);
  }
  for (const Shape& s : list) {
    for (int model = 0; model < 3; ++model) {
      for (int arrival = 0; arrival < 2; ++arrival) {
        if (arrival && (s.split || model == 1)) continue;  // arrival order runs whole tiles
        if (!run_shape(s, model, rng, arrival != 0)) {
          std::printf("FAIL: M=%lld N=%lld W=%d KS=%d BKf=%d BM=%d BK=%d G=%d split=%d model=%d arrival=%d: %s\n",
                      (long long)s.M, (long long)s.N, s.W, s.KS, s.BKf, s.cfg.BM, s.cfg.BK, s.G, (int)s.split, model,
                      arrival, g_fail);
          return 1;
        }
      }
    }
    ++shapes;
  }
  std::printf("ok: %d shapes, %lld checks\n", shapes, g_checks);
  return 0;
}
