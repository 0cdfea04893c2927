// Host-side checks of the DMS library's pure C++ logic (host_logic.h), built
// with the address and undefined-behaviour sanitizers by
// tests/test_host_sanitizers.py: configuration checks, the cache buffer's
// layout, statistics, the serving accounting (worst-case pages of a
// continuation against a brute-force replay of the slot rule) and the
// structural invariant check (consistent tables from random histories pass;
// each planted mistake sets its bit).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "host_logic.h"

using namespace dms;

static int g_fail = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

static dms_config base() {
  dms_config c{};
  c.max_batch = 2;
  c.num_q_heads = 8;
  c.num_kv_heads = 2;
  c.head_dim = 64;
  c.hidden = 256;
  c.window = 16;
  c.block_size = 8;
  c.max_tokens_per_seq = 100;
  c.pool_pages = 32;
  c.max_chunk = 64;
  c.kv_dtype = DMS_BF16;
  c.decide_mode = DMS_DECIDE_LINEAR;
  c.alpha_per = DMS_ALPHA_PER_HEAD;
  c.alpha_scale = 100.0f;
  c.rms_eps = 1e-6f;
  return c;
}

static void check_config() {
  int st = -99;
  dms_config c = base();
  CHECK(config_error(&c, &st) == nullptr && st == DMS_OK);
  CHECK(config_error(nullptr, &st) != nullptr && st == DMS_ERR_ARG);
  struct Case {
    void (*edit)(dms_config&);
    const char* msg;
  };
  const Case cases[] = {
      {[](dms_config& x) { x.block_size = 0; }, "block_size"},
      {[](dms_config& x) { x.window = 8; }, "window must be greater"},
      {[](dms_config& x) { x.num_q_heads = 6; x.num_kv_heads = 4; }, "multiple"},
      {[](dms_config& x) { x.num_q_heads = 24; }, "group size"},
      {[](dms_config& x) { x.head_dim = 96; }, "head_dim"},
      {[](dms_config& x) { x.hidden = 130; }, "hidden"},
      {[](dms_config& x) { x.max_chunk = 10000; }, "max_chunk"},
      {[](dms_config& x) { x.max_batch = 0; }, "positive"},
      {[](dms_config& x) { x.max_batch = 300; x.num_kv_heads = 8; x.num_q_heads = 32; }, "2048"},
      {[](dms_config& x) { x.kv_dtype = 7; }, "kv_dtype"},
      {[](dms_config& x) { x.alpha_per = 2; }, "alpha_per"},
      {[](dms_config& x) { x.decide_mode = 5; }, "decide_mode"},
      {[](dms_config& x) { x.rms_eps = -1.0f; }, "eps"},
      {[](dms_config& x) { x.alpha_scale = NAN; }, "finite"},
      {[](dms_config& x) { x.pool_pages = 1 << 28; }, "2^31"},
      {[](dms_config& x) { x.max_tokens_per_seq = 1 << 30; }, "too large"},
      {[](dms_config& x) { x.num_kv_heads = 32; x.num_q_heads = 32; }, "<= 16"},
  };
  for (const Case& k : cases) {
    dms_config x = base();
    k.edit(x);
    const char* why = config_error(&x, &st);
    CHECK(why != nullptr && st == DMS_ERR_CONFIG && std::strstr(why, k.msg) != nullptr);
  }
}

static void check_layout() {
  std::mt19937 rng(12345);
  auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); };
  for (int it = 0; it < 2000; ++it) {
    dms_config c = base();
    c.num_kv_heads = pick({1, 2, 4, 8, 16});
    c.num_q_heads = c.num_kv_heads * pick({1, 2, 4, 8});
    c.max_batch = 1 + static_cast<int>(rng() % (kMaxUnits / c.num_kv_heads));
    c.head_dim = pick({32, 64, 128});
    c.block_size = pick({1, 7, 16, 256, 1000});
    c.window = c.block_size + 1 + static_cast<int>(rng() % 600);
    c.max_tokens_per_seq = 1 + static_cast<int>(rng() % 40000);
    c.pool_pages = 1 + static_cast<int>(rng() % 5000);
    c.max_chunk = 1 + static_cast<int>(rng() % kMaxChunk);
    c.kv_dtype = pick({DMS_F32, DMS_BF16, DMS_FP8_E4M3});
    c.hidden = 4 * (1 + static_cast<int>(rng() % 2048));
    int st;
    if (config_error(&c, &st)) continue;
    Layout L;
    compute_layout(c, &L);
    const size_t off[] = {L.k_pages, L.v_pages, L.scales, L.page_amax, L.slot_meta, L.page_table, L.lengths, L.ring,
                          L.ring_row, L.cur_page, L.pos, L.free_stack, L.ctl, L.chunk_slot, L.chunk_info,
                          L.unit_info, L.arrive, L.plan, L.decide_w, L.total};
    const size_t units = static_cast<size_t>(c.max_batch) * c.num_kv_heads;
    const size_t maxp = (static_cast<size_t>(c.max_tokens_per_seq) + c.block_size - 1) / c.block_size;
    const size_t pool = c.pool_pages, P = c.block_size;
    const size_t need[] = {pool * P * c.head_dim * kv_elem_bytes(c.kv_dtype),
                           pool * P * c.head_dim * kv_elem_bytes(c.kv_dtype),
                           pool * 8, pool * 8, pool * P * 4, units * maxp * 4, units * 4,
                           units * c.window * 4, units * c.window * 4, units * 4, static_cast<size_t>(c.max_batch) * 4,
                           pool * 4, kCtlWords * 4, units * c.max_chunk * 4, units * 32, kMaxUnits * 16,
                           kArriveGroups * kArriveStride * 4, plan_words(c.max_batch) * 4,
                           decide_w_bytes(c.hidden)};
    CHECK(L.k_pages == 0);
    for (int r = 0; r < 19; ++r) {
      CHECK(off[r] % 256 == 0);
      CHECK(off[r + 1] >= off[r] + need[r]);          // no region overlaps the next
      CHECK(off[r + 1] - off[r] < need[r] + 256);     // and no more than alignment in between
    }
  }
}

static void check_stats_and_info() {
  std::mt19937 rng(7);
  for (int it = 0; it < 200; ++it) {
    const int Bmax = 1 + rng() % 40, Hkv = 1 + rng() % 16, P = 1 + rng() % 300;
    std::vector<int32_t> len(static_cast<size_t>(Bmax) * Hkv), pos(Bmax);
    for (auto& v : pos) v = rng() % 20000;
    for (int b = 0; b < Bmax; ++b)
      for (int k = 0; k < Hkv; ++k) len[b * Hkv + k] = pos[b] ? static_cast<int32_t>(rng() % (pos[b] + 1)) : 0;
    dms_stats s;
    const int64_t rb = 256;
    stats_from_tables(Bmax, Hkv, P, rb, len.data(), pos.data(), &s);
    int64_t tok = 0, live = 0, pages = 0;
    for (int b = 0; b < Bmax; ++b) {
      tok += static_cast<int64_t>(pos[b]) * Hkv;
      const dms_seq_info si = seq_info_from_tables(b, Hkv, P, len.data(), pos.data());
      int64_t sl = 0, sp = 0, mx = 0;
      for (int k = 0; k < Hkv; ++k) {
        const int64_t L = len[b * Hkv + k];
        sl += L;
        sp += (L + P - 1) / P;
        mx = L > mx ? L : mx;
      }
      CHECK(si.position == pos[b] && si.live_slots == sl && si.pages == sp && si.max_head_slots == mx);
      live += sl;
      pages += sp;
    }
    CHECK(s.tokens == tok && s.live_slots == live && s.pages_in_use == pages);
    CHECK(s.bytes_live == live * rb * 2 && s.bytes_allocated == pages * P * rb * 2);
    CHECK(live == 0 ? s.cache_cr == 0.0 : std::fabs(s.cache_cr - double(tok) / double(live)) < 1e-12);
  }
}

// Replays the slot rule (a token w positions after a marked one takes its
// slot in place, any other token a new slot) over a random history of one
// head, then appends n kept tokens; returns the pages the continuation adds.
static void replay(int w, int P, const std::vector<int>& marks, int n, int32_t* len_out, std::vector<int32_t>* ring,
                   int64_t* pages_added) {
  const int t0 = static_cast<int>(marks.size());
  std::vector<int> slot(t0 + n), mark(marks);
  mark.resize(t0 + n, 0);
  int64_t L = 0;
  for (int t = 0; t < t0 + n; ++t) {
    if (t >= w && mark[t - w]) slot[t] = slot[t - w];
    else slot[t] = static_cast<int>(L++);
    if (t == t0 - 1) *len_out = static_cast<int32_t>(L);
  }
  if (t0 == 0) *len_out = 0;
  ring->assign(w, 0);
  for (int t = (t0 > w ? t0 - w : 0); t < t0; ++t)
    (*ring)[t % w] = static_cast<int32_t>(static_cast<uint32_t>(slot[t]) | (static_cast<uint32_t>(mark[t]) << 31));
  const int64_t L0 = *len_out;
  *pages_added = (L + P - 1) / P - (L0 + P - 1) / P;
}

static void check_worst_pages() {
  std::mt19937 rng(99);
  for (int it = 0; it < 3000; ++it) {
    const int P = 1 + rng() % 8;
    const int w = P + 1 + rng() % 9;
    const int t0 = rng() % 60, n = rng() % 40;
    const double p = (rng() % 100) / 100.0;
    std::vector<int> marks(t0);
    for (auto& m : marks) m = (rng() % 1000) < p * 1000 ? 1 : 0;
    int32_t len = 0;
    std::vector<int32_t> ring;
    int64_t want = 0;
    replay(w, P, marks, n, &len, &ring, &want);
    const int32_t pos = t0;
    const int max_tokens = t0 + n + static_cast<int>(rng() % 3);
    CHECK(worst_pages_for_seq(0, n, 1, w, P, max_tokens, &len, &pos, ring.data()) == want);
    CHECK(worst_pages_for_seq(0, n, 1, w, P, t0 + n - 1, &len, &pos, ring.data()) == -1);   // one past capacity
  }
}

// A consistent set of cache tables built from random histories (the slot
// rule applied token by token, pages popped 0, 1, 2, ... from the pool), then
// one planted mistake per kind of invariant.
struct Tables {
  int Bmax = 2, Hkv = 2, w = 5, P = 3, maxp = 0, pool = 64;
  std::vector<int32_t> len, pt, meta, ring, ring_row, cur, pos, fs;
  int32_t free_count = 0;
  TableView view() const {
    return TableView{Bmax, Hkv, w, P, maxp, pool, len.data(), pt.data(), meta.data(), ring.data(),
                     ring_row.data(), cur.data(), pos.data(), fs.data(), free_count};
  }
};

static Tables build_tables(std::mt19937& rng) {
  Tables t;
  const int max_tokens = 40;
  t.maxp = (max_tokens + t.P - 1) / t.P;
  const int units = t.Bmax * t.Hkv;
  t.len.assign(units, 0);
  t.pt.assign(static_cast<size_t>(units) * t.maxp, -1);
  t.meta.assign(static_cast<size_t>(t.pool) * t.P, 0);
  t.ring.assign(static_cast<size_t>(units) * t.w, 0);
  t.ring_row.assign(static_cast<size_t>(units) * t.w, 0);
  t.cur.assign(units, -1);
  t.pos.assign(t.Bmax, 0);
  int next_page = 0;
  for (int seq = 0; seq < t.Bmax; ++seq) {
    const int T = static_cast<int>(rng() % (max_tokens + 1));
    t.pos[seq] = T;
    for (int k = 0; k < t.Hkv; ++k) {
      const int unit = seq * t.Hkv + k;
      std::vector<int> slot(T), mark(T);
      int L = 0;
      for (int p = 0; p < T; ++p) {
        mark[p] = static_cast<int>(rng() % 2);
        if (p >= t.w && mark[p - t.w]) {
          slot[p] = slot[p - t.w];
        } else {
          slot[p] = L++;
          if ((L - 1) % t.P == 0) t.pt[static_cast<size_t>(unit) * t.maxp + (L - 1) / t.P] = next_page++;
        }
        const int row = t.pt[static_cast<size_t>(unit) * t.maxp + slot[p] / t.P] * t.P + slot[p] % t.P;
        t.meta[row] = static_cast<int32_t>(static_cast<uint32_t>(p) | (static_cast<uint32_t>(mark[p]) << 31));
        t.ring[static_cast<size_t>(unit) * t.w + p % t.w] =
            static_cast<int32_t>(static_cast<uint32_t>(slot[p]) | (static_cast<uint32_t>(mark[p]) << 31));
        t.ring_row[static_cast<size_t>(unit) * t.w + p % t.w] = row;
      }
      t.len[unit] = L;
      if (L > 0) t.cur[unit] = t.pt[static_cast<size_t>(unit) * t.maxp + (L - 1) / t.P];
    }
  }
  for (int pg = t.pool - 1; pg >= next_page; --pg) t.fs.push_back(pg);
  t.free_count = static_cast<int32_t>(t.fs.size());
  t.fs.resize(t.pool, 0);
  return t;
}

static void check_invariants() {
  std::mt19937 rng(4242);
  int planted = 0;
  for (int it = 0; it < 500; ++it) {
    Tables t = build_tables(rng);
    int where = 0;
    CHECK(check_tables(t.view(), &where) == 0 && where == -1);
    // the longest head, for mistakes that need live slots
    int u = 0;
    for (int i = 1; i < t.Bmax * t.Hkv; ++i)
      if (t.len[i] > t.len[u]) u = i;
    const int L = t.len[u], T = t.pos[u / t.Hkv];
    if (L < 2 || T <= t.w) continue;
    ++planted;
    int32_t* ptu = t.pt.data() + static_cast<size_t>(u) * t.maxp;
    {  // a page held twice
      Tables x = t;
      int v = u == 0 ? 1 : 0;
      if (x.len[v] > 0) {
        x.pt[static_cast<size_t>(v) * x.maxp] = ptu[0];
        CHECK(check_tables(x.view(), &where) & kChkOwnership);
      }
    }
    {  // a page lost (one fewer free)
      Tables x = t;
      if (x.free_count > 0) {
        x.free_count -= 1;
        CHECK(check_tables(x.view(), &where) & kChkOwnership);
      }
    }
    {  // a page id outside the pool
      Tables x = t;
      x.pt[static_cast<size_t>(u) * x.maxp] = x.pool;
      CHECK((check_tables(x.view(), &where) & kChkPageId) && where == u);
    }
    {  // a live slot holding a token that left the window marked: use the
       // position of a slot's second occupant minus w (the overwritten one)
      Tables x = t;
      bool done = false;
      for (int s = 0; s < L && !done; ++s) {
        const int row = ptu[s / x.P] * x.P + s % x.P;
        const int p = static_cast<int>(static_cast<uint32_t>(x.meta[row]) & 0x7FFFFFFFu);
        if (p >= x.w) {
          // position p - w: marked (its slot was reused) or kept elsewhere
          x.meta[row] = static_cast<int32_t>(static_cast<uint32_t>(p - x.w) | (1u << 31));
          if ((T - 1) - (p - x.w) >= x.w) {
            CHECK((check_tables(x.view(), &where) & kChkSlot) && where == u);
            done = true;
          } else {
            x.meta[row] = t.meta[row];
          }
        }
      }
    }
    {  // two slots holding the same token
      Tables x = t;
      const int r0 = ptu[0] * x.P, r1 = ptu[1 / x.P] * x.P + 1 % x.P;
      x.meta[r1] = x.meta[r0];
      CHECK(check_tables(x.view(), &where) & (kChkSlot | kChkRing));
    }
    {  // a window entry naming another slot
      Tables x = t;
      const size_t ri = static_cast<size_t>(u) * x.w + static_cast<size_t>((T - 1) % x.w);
      const uint32_t e = static_cast<uint32_t>(x.ring[ri]);
      const uint32_t s2 = ((e & 0x7FFFFFFFu) + 1) % static_cast<uint32_t>(L);
      x.ring[ri] = static_cast<int32_t>(s2 | (e & 0x80000000u));
      CHECK((check_tables(x.view(), &where) & kChkRing) && where == u);
    }
    {  // a wrong current page
      Tables x = t;
      x.cur[u] = x.pool + 5;
      CHECK((check_tables(x.view(), &where) & kChkCurPage) && where == u);
    }
    {  // a length past the position
      Tables x = t;
      x.len[u] = T + 1;
      CHECK(check_tables(x.view(), &where) & kChkLength);
    }
    {  // a bad free count
      Tables x = t;
      x.free_count = x.pool + 1;
      CHECK(check_tables(x.view(), &where) & kChkFreeStack);
    }
  }
  CHECK(planted > 100);
}

int main() {
  check_invariants();
  check_config();
  check_layout();
  check_stats_and_info();
  check_worst_pages();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks ok\n");
  return 0;
}
