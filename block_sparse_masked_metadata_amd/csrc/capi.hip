// C ABI of libbsm.so (declared in include/bsm.h): argument checks, device-plan
// packing and launch wrappers.  No device memory is allocated here; every
// device buffer belongs to the caller.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "kernels.hpp"
#include "planner.hpp"

namespace bsm {

namespace {
thread_local std::string g_error;

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("BSM_DEBUG_SYNC");
    return e && e[0] == '1';
  }();
  return on;
}

int hip_status(hipError_t e, const char* what, hipStream_t stream) {
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return BSM_E_HIP;
  }
  return BSM_OK;
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

struct StepLists {
  std::vector<int4> fitems, bitems;
  std::vector<int4> citems;  // fitems by chain: chain 0's items first (bsm_fwd_step_chain)
  int64_t nchain0 = 0;
  std::vector<int4> bwork, breduce;  // split dK/dV work and its reduction
  int32_t slots = 0;                 // workspace slots of the split work
  int64_t pairs = 0;
};
}  // namespace

void set_error(const std::string& msg) { g_error = msg; }

// Host image of one rank's device plan.
struct Packed {
  std::vector<int4> tracks;
  std::vector<int32_t> coord;  // per plan row: its token index in the caller's order
  std::vector<StepLists> steps;
  std::vector<int4> sitems;
  std::vector<int2> kint;  // key intervals (lo, hi) in plan order
  // sparse fetch: one pass over [local shard | needed remote tiles]
  std::vector<int4> xitems, xtracks;
  std::vector<int2> xkint;
  std::vector<int4> yitems;   // the fetched pass's dK/dV column items (compact key tiles)
  std::vector<int32_t> xsrc;  // shard row (plan order) of each compact row, -1 for padding
  int64_t fetch_tiles = 0, fetch_rows = 0;
  std::vector<int2> entries;
  // byte offsets in the device buffer
  int64_t off_tracks = 0, off_coord = 0, off_kint = 0, off_items = 0, off_entries = 0, bytes = 0;
  std::vector<int64_t> off_f, off_b, off_ff;  // off_ff: first list entry of each forward item
  std::vector<int64_t> off_c, off_cf;         // the chain-ordered forward items and their first entries
  std::vector<int64_t> off_w, off_r;         // split dK/dV work units and reduce entries
  int64_t off_s = 0, off_sf = 0, off_x = 0, off_xf = 0, off_xtracks = 0, off_xkint = 0;
  int64_t off_y = 0, off_xsrc = 0;
};

static void layout(const Plan& p, Packed& pk);

// Split work of one step's dK/dV items (one workgroup per item and kv head
// lasts as long as its column list): a list longer than the mean is cut into
// sub-tile ranges of about the mean length (at most 16); the first range adds
// into dK/dV, each other one writes a workspace slot that a reduction adds
// in slot order afterwards.  Units longest first.
static void split_work(StepLists& st) {
  st.bwork.clear();
  st.breduce.clear();
  st.slots = 0;
  if (st.bitems.empty()) return;
  int64_t sum = 0;
  for (const int4& it : st.bitems) sum += 2 * (int64_t)it.w;
  const int64_t n_items = (int64_t)st.bitems.size();
  const int32_t L = (int32_t)std::max<int64_t>(4, (sum + n_items - 1) / n_items);
  for (int32_t i = 0; i < (int32_t)n_items; ++i) {
    const int32_t n = 2 * st.bitems[i].w;
    const int32_t parts = std::min<int32_t>(16, (n + L - 1) / L);
    if (parts <= 1) {
      st.bwork.push_back(make_int4(i, 0, n, -1));
      continue;
    }
    st.breduce.push_back(make_int4(st.bitems[i].x, st.slots, parts - 1, key_rows(st.bitems[i].y)));
    for (int32_t q = 0; q < parts; ++q) {
      const int32_t a0 = (int32_t)((int64_t)n * q / parts), a1 = (int32_t)((int64_t)n * (q + 1) / parts);
      st.bwork.push_back(make_int4(i, a0, a1, q == 0 ? -1 : st.slots++));
    }
  }
  std::stable_sort(st.bwork.begin(), st.bwork.end(),
                   [](const int4& x, const int4& y) { return x.z - x.y > y.z - y.y; });
}

// Work items longest list first, then grouped by the sample of their tile's
// first row, groups in the order of their longest item: items of one sample
// read the same key tiles, so a group's tiles stay in the L2 of each XCD
// while it runs (on the 64K multimodal share 16% fewer bytes read per step;
// the longest-first order alone lets a sample's items drift apart and its key
// tiles be fetched 1.6 times).
template <class G>
static void order_items(std::vector<int4>& v, G group) {
  std::stable_sort(v.begin(), v.end(), [](const int4& x, const int4& y) { return x.w != y.w ? x.w > y.w : x.x < y.x; });
  std::vector<std::pair<int32_t, int32_t>> rank;  // (group, first position)
  std::vector<int32_t> key(v.size());
  for (size_t i = 0; i < v.size(); ++i) {
    const int32_t g = group(v[i].x);
    auto it = std::find_if(rank.begin(), rank.end(), [&](const std::pair<int32_t, int32_t>& e) { return e.first == g; });
    if (it == rank.end()) {
      rank.push_back({g, (int32_t)rank.size()});
      key[i] = rank.back().second;
    } else {
      key[i] = it->second;
    }
  }
  std::vector<size_t> idx(v.size());
  for (size_t i = 0; i < idx.size(); ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) { return key[a] < key[b]; });
  std::vector<int4> out(v.size());
  for (size_t i = 0; i < idx.size(); ++i) out[i] = v[idx[i]];
  v.swap(out);
}

// Two chains of query tiles for the forward (bsm_fwd_step_chain): a step's
// items of one chain depend only on that chain's items of earlier steps, so
// the two chains can run on two streams and fill each other's launch tails.
// Whole samples (the sample of a tile's first row) go to one chain, so a
// chain keeps order_items' grouping of a sample's items; heaviest sample
// first to the lighter chain, weighed by list entries over all steps, ties
// by sample id.  Each step's items in chain order, order_items' order kept
// within a chain.
template <class W, class G>
static void chain_items(Packed& pk, int32_t T, int32_t R, W entries_of, G group) {
  std::vector<std::pair<int32_t, int64_t>> gw;  // (sample, list entries)
  for (int32_t a = 0; a < T; ++a) {
    int64_t w = 0;
    for (int32_t s = 0; s < R; ++s) w += entries_of(s, a);
    if (w == 0) continue;
    const int32_t g = group(a);
    auto it = std::find_if(gw.begin(), gw.end(), [&](const std::pair<int32_t, int64_t>& e) { return e.first == g; });
    if (it == gw.end()) gw.push_back({g, w});
    else it->second += w;
  }
  std::sort(gw.begin(), gw.end(), [](const std::pair<int32_t, int64_t>& x, const std::pair<int32_t, int64_t>& y) {
    return x.second != y.second ? x.second > y.second : x.first < y.first;
  });
  std::vector<std::pair<int32_t, int32_t>> gc;  // (sample, chain)
  int64_t load[2] = {0, 0};
  for (const auto& e : gw) {
    const int32_t c = load[1] < load[0] ? 1 : 0;
    gc.push_back({e.first, c});
    load[c] += e.second;
  }
  auto chain_of = [&](int32_t a) {
    const int32_t g = group(a);
    for (const auto& e : gc)
      if (e.first == g) return e.second;
    return 0;
  };
  for (int32_t s = 0; s < R; ++s) {
    StepLists& st = pk.steps[s];
    st.citems = st.fitems;
    auto mid = std::stable_partition(st.citems.begin(), st.citems.end(),
                                     [&](const int4& x) { return chain_of(x.x) == 0; });
    st.nchain0 = mid - st.citems.begin();
  }
}

static void pack(const Plan& p, int32_t r, Packed& pk) {
  const int32_t R = p.ranks, T = p.tps;
  const int64_t S = p.shard;
  pk.tracks.resize(p.n);
  pk.kint.resize(p.n);
  pk.coord.assign(p.perm.begin(), p.perm.end());
  for (int64_t i = 0; i < p.n; ++i) {
    const int32_t t = p.perm[i];
    pk.tracks[i] = make_int4(p.sample[t], p.seg[t], p.noise[t], p.pos[t]);
    pk.kint[i] = make_int2(p.klo[t], p.khi[t]);
  }
  // a partner key tile (local tile b of shard j) whose keys all have intervals
  auto kint_tile = [&](int32_t j, int32_t b) { return p.tile_kint[p.tiles_new[(int64_t)j * T + b]] != 0; };
  auto tlen = [&](int32_t a) { return (int32_t)std::min<int64_t>(kTile, S - (int64_t)a * kTile); };
  // sample of the first row of query tile a of rank r
  auto qsample = [&](int32_t a) { return p.sample[p.perm[(int64_t)r * S + (int64_t)a * kTile]]; };
  // per step row lists: rows[s][a] = (b, class) ascending b
  std::vector<std::vector<std::vector<std::pair<int32_t, uint8_t>>>> rows(
      R, std::vector<std::vector<std::pair<int32_t, uint8_t>>>(T));
  std::vector<int64_t> step_pairs(R, 0);
  for (int32_t a = 0; a < T; ++a) {
    const int32_t tq = p.tiles_new[(int64_t)r * T + a];
    for (int64_t e = p.pptr[tq]; e < p.pptr[tq + 1]; ++e) {
      const int32_t tk = p.pkey[e];
      const int32_t j = p.owner[tk];
      const int32_t s = ((r - j) % R + R) % R;
      rows[s][a].push_back({p.local[tk], p.pclass[e]});
      step_pairs[s] += p.pcount[e];
    }
  }
  std::vector<int32_t> first(T, -1), last(T, -1);
  for (int32_t s = 0; s < R; ++s)
    for (int32_t a = 0; a < T; ++a) {
      std::sort(rows[s][a].begin(), rows[s][a].end());
      if (!rows[s][a].empty()) {
        if (first[a] < 0) first[a] = s;
        last[a] = s;
      }
    }
  auto by_len = [](const int4& x, const int4& y) { return x.w != y.w ? x.w > y.w : x.x < y.x; };
  pk.steps.assign(R, StepLists());
  pk.entries.clear();
  for (int32_t s = 0; s < R; ++s) {
    StepLists& st = pk.steps[s];
    st.pairs = step_pairs[s];
    // forward / dQ: query-tile major
    for (int32_t a = 0; a < T; ++a) {
      if (rows[s][a].empty()) continue;
      const int32_t flags = (first[a] == s ? kFirst : 0) | (last[a] == s ? kLast : 0);
      st.fitems.push_back(make_int4(a, flags, (int32_t)pk.entries.size(), (int32_t)rows[s][a].size()));
      const int32_t j = ((r - s) % R + R) % R;
      for (auto& bc : rows[s][a]) {
        const int32_t kl = tlen(bc.first);
        const bool part = bc.second == BSM_TILE_PARTIAL || kl < kTile;
        const bool kin = part && kint_tile(j, bc.first);
        pk.entries.push_back(make_int2(bc.first * kTile, kl | (part ? kPartialBit : 0) | (kin ? kIntervalBit : 0)));
      }
    }
    order_items(st.fitems, qsample);
    // dK/dV: key-tile major (column lists, ascending query tile)
    std::vector<std::vector<std::pair<int32_t, uint8_t>>> cols(T);
    for (int32_t a = 0; a < T; ++a)
      for (auto& bc : rows[s][a]) cols[bc.first].push_back({a, bc.second});
    for (int32_t b = 0; b < T; ++b) {
      if (cols[b].empty()) continue;
      const int32_t jb = ((r - s) % R + R) % R;
      st.bitems.push_back(make_int4(b * kTile, (kint_tile(jb, b) ? kKeyInterval : 0) | (tlen(b) << kKeyRowsShift),
                                    (int32_t)pk.entries.size(), (int32_t)cols[b].size()));
      for (auto& ac : cols[b]) {
        const int32_t ql = tlen(ac.first);
        const bool part = ac.second == BSM_TILE_PARTIAL || ql < kTile;
        pk.entries.push_back(make_int2(ac.first * kTile, ql | (part ? kPartialBit : 0)));
      }
    }
    std::stable_sort(st.bitems.begin(), st.bitems.end(), by_len);
    split_work(st);
  }
  chain_items(pk, T, R, [&](int32_t s, int32_t a) { return (int64_t)rows[s][a].size(); }, qsample);
  // merged single-pass lists: ring step order, then ascending key tile
  pk.sitems.clear();
  for (int32_t a = 0; a < T; ++a) {
    const int32_t beg = (int32_t)pk.entries.size();
    for (int32_t s = 0; s < R; ++s) {
      const int32_t j = ((r - s) % R + R) % R;
      for (auto& bc : rows[s][a]) {
        const int32_t kl = tlen(bc.first);
        const bool part = bc.second == BSM_TILE_PARTIAL || kl < kTile;
        const bool kin = part && kint_tile(j, bc.first);
        pk.entries.push_back(make_int2((int32_t)(j * S + (int64_t)bc.first * kTile),
                                       kl | (part ? kPartialBit : 0) | (kin ? kIntervalBit : 0)));
      }
    }
    const int32_t cnt = (int32_t)pk.entries.size() - beg;
    if (cnt) pk.sitems.push_back(make_int4(a, kFirst | kLast, beg, cnt));
  }
  order_items(pk.sitems, qsample);

  // sparse fetch: the local shard, then the needed remote key tiles in ring
  // step order (s = 1 .. R-1), ascending tile; each remote tile takes 128 rows
  {
    std::vector<uint8_t> need((size_t)R * T);
    pk.fetch_tiles = fetch_set(p, r, need.data());
    std::vector<int64_t> slot((size_t)R * T, -1);
    for (int32_t b = 0; b < T; ++b) slot[(size_t)r * T + b] = (int64_t)b * kTile;
    int64_t next = S;
    for (int32_t s = 1; s < R; ++s) {
      const int32_t j = ((r - s) % R + R) % R;
      for (int32_t b = 0; b < T; ++b)
        if (need[(size_t)j * T + b]) {
          slot[(size_t)j * T + b] = next;
          next += kTile;
        }
    }
    pk.fetch_rows = next;
    pk.xtracks.assign(next, make_int4(-1, -1, -1, 0));
    pk.xkint.assign(next, make_int2(0, -1));
    pk.xsrc.assign(next, -1);
    for (int32_t j = 0; j < R; ++j)
      for (int32_t b = 0; b < T; ++b) {
        const int64_t base = slot[(size_t)j * T + b];
        if (base < 0) continue;
        for (int32_t i = 0; i < tlen(b); ++i) {
          pk.xtracks[base + i] = pk.tracks[(int64_t)j * S + (int64_t)b * kTile + i];
          pk.xkint[base + i] = pk.kint[(int64_t)j * S + (int64_t)b * kTile + i];
          pk.xsrc[base + i] = (int32_t)((int64_t)j * S + (int64_t)b * kTile + i);
        }
      }
    pk.xitems.clear();
    for (int32_t a = 0; a < T; ++a) {
      const int32_t beg = (int32_t)pk.entries.size();
      for (int32_t s = 0; s < R; ++s) {
        const int32_t j = ((r - s) % R + R) % R;
        for (auto& bc : rows[s][a]) {
          const int32_t kl = tlen(bc.first);
          const bool part = bc.second == BSM_TILE_PARTIAL || kl < kTile;
          const bool kin = part && kint_tile(j, bc.first);
          pk.entries.push_back(make_int2((int32_t)slot[(size_t)j * T + bc.first],
                                         kl | (part ? kPartialBit : 0) | (kin ? kIntervalBit : 0)));
        }
      }
      const int32_t cnt = (int32_t)pk.entries.size() - beg;
      if (cnt) pk.xitems.push_back(make_int4(a, kFirst | kLast, beg, cnt));
    }
    order_items(pk.xitems, qsample);
    // dK/dV over the compact buffer: per compact key tile, its query tiles
    // in ascending order (one pass, every step's pairs of that tile)
    pk.yitems.clear();
    for (int32_t s = 0; s < R; ++s) {
      const int32_t j = ((r - s) % R + R) % R;
      std::vector<std::vector<std::pair<int32_t, uint8_t>>> cols(T);
      for (int32_t a = 0; a < T; ++a)
        for (auto& bc : rows[s][a]) cols[bc.first].push_back({a, bc.second});
      for (int32_t b = 0; b < T; ++b) {
        if (cols[b].empty()) continue;
        const int64_t base = slot[(size_t)j * T + b];
        pk.yitems.push_back(make_int4((int32_t)base,
                                      (kint_tile(j, b) ? kKeyInterval : 0) | (tlen(b) << kKeyRowsShift),
                                      (int32_t)pk.entries.size(), (int32_t)cols[b].size()));
        for (auto& ac : cols[b]) {
          const int32_t ql = tlen(ac.first);
          const bool part = ac.second == BSM_TILE_PARTIAL || ql < kTile;
          pk.entries.push_back(make_int2(ac.first * kTile, ql | (part ? kPartialBit : 0)));
        }
      }
    }
    std::stable_sort(pk.yitems.begin(), pk.yitems.end(), by_len);
  }

  layout(p, pk);
}

// Byte layout of the device image.
static void layout(const Plan& p, Packed& pk) {
  const int32_t R = p.ranks;
  int64_t off = 0;
  pk.off_tracks = off;
  off = align256(off + p.n * (int64_t)sizeof(int4));
  pk.off_coord = off;
  off = align256(off + p.n * (int64_t)sizeof(int32_t));
  pk.off_kint = off;
  off = align256(off + p.n * (int64_t)sizeof(int2));
  pk.off_items = off;
  pk.off_f.assign(R, 0);
  pk.off_b.assign(R, 0);
  pk.off_ff.assign(R, 0);
  pk.off_c.assign(R, 0);
  pk.off_cf.assign(R, 0);
  pk.off_w.assign(R, 0);
  pk.off_r.assign(R, 0);
  for (int32_t s = 0; s < R; ++s) {
    pk.off_f[s] = off;
    off = align256(off + (int64_t)pk.steps[s].fitems.size() * sizeof(int4));
    pk.off_ff[s] = off;
    off = align256(off + (int64_t)pk.steps[s].fitems.size() * sizeof(int2));
    pk.off_c[s] = off;
    off = align256(off + (int64_t)pk.steps[s].citems.size() * sizeof(int4));
    pk.off_cf[s] = off;
    off = align256(off + (int64_t)pk.steps[s].citems.size() * sizeof(int2));
    pk.off_b[s] = off;
    off = align256(off + (int64_t)pk.steps[s].bitems.size() * sizeof(int4));
    pk.off_w[s] = off;
    off = align256(off + (int64_t)pk.steps[s].bwork.size() * sizeof(int4));
    pk.off_r[s] = off;
    off = align256(off + (int64_t)pk.steps[s].breduce.size() * sizeof(int4));
  }
  pk.off_s = off;
  off = align256(off + (int64_t)pk.sitems.size() * sizeof(int4));
  pk.off_sf = off;
  off = align256(off + (int64_t)pk.sitems.size() * sizeof(int2));
  pk.off_x = off;
  off = align256(off + (int64_t)pk.xitems.size() * sizeof(int4));
  pk.off_xf = off;
  off = align256(off + (int64_t)pk.xitems.size() * sizeof(int2));
  pk.off_xtracks = off;
  off = align256(off + pk.fetch_rows * (int64_t)sizeof(int4));
  pk.off_xkint = off;
  off = align256(off + pk.fetch_rows * (int64_t)sizeof(int2));
  pk.off_y = off;
  off = align256(off + (int64_t)pk.yitems.size() * sizeof(int4));
  pk.off_xsrc = off;
  off = align256(off + (int64_t)pk.xsrc.size() * sizeof(int32_t));
  pk.off_entries = off;
  off = align256(off + (int64_t)pk.entries.size() * sizeof(int2));
  pk.bytes = std::max<int64_t>(off, 256);
}

// Position bounds of local rows [a, b) of the shard at plan row `base`;
// positions rise within each 128-row tile of a shard.
static void row_bounds(const Plan& p, int64_t base, int64_t a, int64_t b, int64_t& mn, int64_t& mx) {
  mn = INT64_MAX;
  mx = INT64_MIN;
  for (int64_t x = a; x < b;) {
    const int64_t y = std::min<int64_t>(b, (x / kTile + 1) * kTile);
    mn = std::min<int64_t>(mn, p.pos[p.perm[base + x]]);
    mx = std::max<int64_t>(mx, p.pos[p.perm[base + y - 1]]);
    x = y;
  }
}

namespace {
struct DenseEnt {
  int32_t k0, kl, qlo, qhi, kind;
  int64_t qmin, qmax, kmin, kmax;
};
}  // namespace

// Dense-call lists of rank r (MARBLE section 03, "Chunked ring attention"):
// each call of a step becomes, per query tile it meets, one list entry per
// key tile its key run meets, carrying the call's relation and the tile rows
// it applies to; pieces no pair of which satisfies the relation are dropped,
// pieces every pair of which does become full.  Entries of one tile with the
// same rows and keys whose relations leave no pair out merge into one full
// entry.  Returns BSM_OK or an error code.
static int pack_calls(const Plan& p, int32_t r, Packed& pk) {
  const int32_t R = p.ranks, T = p.tps;
  const int64_t S = p.shard;
  if (p.pos[p.n - 1] >= INT32_MAX) {
    set_error("dense calls need positions below 2^31 - 1");
    return BSM_E_UNSUPPORTED;
  }
  pk.tracks.resize(p.n);
  pk.kint.assign(p.n, make_int2(0, -1));
  pk.coord.assign(p.perm.begin(), p.perm.end());
  for (int64_t i = 0; i < p.n; ++i) {
    const int32_t t = p.perm[i];
    pk.tracks[i] = make_int4(p.sample[t], p.seg[t], p.noise[t], p.pos[t]);
  }
  std::vector<std::vector<std::vector<int2>>> lists(R, std::vector<std::vector<int2>>(T));
  std::vector<Call> calls;
  std::vector<std::vector<DenseEnt>> per_tile(T);
  pk.steps.assign(R, StepLists());
  for (int32_t s = 0; s < R; ++s) {
    const int32_t j = ((r - s) % R + R) % R;
    const int64_t qbase = (int64_t)r * S, kbase = (int64_t)j * S;
    int rc = dense_calls(p, r, s, calls);
    if (rc) return rc;
    for (auto& v : per_tile) v.clear();
    for (const Call& c : calls) {
      // the call's key pieces: its key run cut at key-tile edges, so each
      // piece is one column entry of one key tile in the dK/dV lists
      std::vector<std::pair<int32_t, int32_t>> kp;  // [first row, end)
      std::vector<std::pair<int64_t, int64_t>> kb;  // position bounds
      for (int32_t b = c.k0 / kTile; b <= (c.k0 + c.kn - 1) / kTile; ++b) {
        const int32_t k = std::max(c.k0, b * kTile), ke = std::min(c.k0 + c.kn, (b + 1) * kTile);
        int64_t mn, mx;
        row_bounds(p, kbase, k, ke, mn, mx);
        kp.push_back({k, ke});
        kb.push_back({mn, mx});
      }
      for (int32_t a = c.q0 / kTile; a <= (c.q0 + c.qn - 1) / kTile; ++a) {
        const int32_t ra = std::max(c.q0, a * kTile), rb = std::min(c.q0 + c.qn, (a + 1) * kTile);
        int64_t qmn, qmx;
        row_bounds(p, qbase, ra, rb, qmn, qmx);
        for (size_t i = 0; i < kb.size(); ++i) {
          const int cls = relation_bounds(c.kind, qmn, qmx, kb[i].first, kb[i].second, p.window);
          if (cls == 0) continue;
          per_tile[a].push_back({kp[i].first, kp[i].second - kp[i].first, ra - a * kTile, rb - a * kTile,
                                 cls == 2 ? (int32_t)kCallFull : c.kind, qmn, qmx, kb[i].first, kb[i].second});
        }
      }
    }
    for (int32_t a = 0; a < T; ++a) {
      auto& v = per_tile[a];
      std::sort(v.begin(), v.end(), [](const DenseEnt& x, const DenseEnt& y) {
        return std::tie(x.k0, x.kl, x.qlo, x.qhi, x.kind) < std::tie(y.k0, y.kl, y.qlo, y.qhi, y.kind);
      });
      const int32_t tile_rows = (int32_t)std::min<int64_t>(kTile, S - (int64_t)a * kTile);
      for (size_t g = 0; g < v.size();) {
        size_t h = g + 1;
        while (h < v.size() && v[h].k0 == v[g].k0 && v[h].kl == v[g].kl && v[h].qlo == v[g].qlo &&
               v[h].qhi == v[g].qhi)
          ++h;
        // relations present; the group is full when every absent one has no pair
        bool full = h - g > 1;
        if (full) {
          uint32_t mask = 0;
          for (size_t i = g; i < h; ++i) mask |= 1u << v[i].kind;
          if (mask & (1u << kCallFull)) full = false;
          for (int32_t kd : {(int32_t)kCallCausal, (int32_t)kCallReverse, (int32_t)kCallPastWindow})
            if (full && !(mask & (1u << kd)) &&
                relation_bounds(kd, v[g].qmin, v[g].qmax, v[g].kmin, v[g].kmax, p.window) != 0)
              full = false;
        }
        for (size_t i = g; i < (full ? g + 1 : h); ++i) {
          const DenseEnt& e = v[i];
          const int32_t kind = full ? (int32_t)kCallFull : e.kind;
          const bool whole = e.qlo == 0 && e.qhi == tile_rows;
          const bool part = !(kind == kCallFull && whole && e.kl == kTile);
          lists[s][a].push_back(make_int2(e.k0, e.kl | (e.qlo << kRowLoShift) | ((e.qhi - 1) << kRowHiShift) |
                                                    (kind << kKindShift) | (part ? kPartialBit : 0)));
        }
        g = h;
      }
    }
  }
  auto qsample = [&](int32_t a) { return p.sample[p.perm[(int64_t)r * S + (int64_t)a * kTile]]; };
  std::vector<int32_t> first(T, -1), last(T, -1);
  for (int32_t s = 0; s < R; ++s)
    for (int32_t a = 0; a < T; ++a)
      if (!lists[s][a].empty()) {
        if (first[a] < 0) first[a] = s;
        last[a] = s;
      }
  pk.entries.clear();
  for (int32_t s = 0; s < R; ++s) {
    StepLists& st = pk.steps[s];
    st.pairs = step_map(p, r, s, nullptr);
    for (int32_t a = 0; a < T; ++a) {
      if (lists[s][a].empty()) continue;
      const int32_t flags = (first[a] == s ? kFirst : 0) | (last[a] == s ? kLast : 0);
      st.fitems.push_back(make_int4(a, flags, (int32_t)pk.entries.size(), (int32_t)lists[s][a].size()));
      pk.entries.insert(pk.entries.end(), lists[s][a].begin(), lists[s][a].end());
    }
    order_items(st.fitems, qsample);
    // dK/dV column lists: every row entry, cut at key-tile edges, becomes an
    // entry of each key tile it meets (x = first query row, the key rows of
    // the tile it applies to in the row bits), ascending query row.  Query
    // rows past a column entry's length carry P = 0 (LSE = -inf), so only key
    // coverage and the relation decide whether it is masked.
    std::vector<std::vector<int2>> cols(T);
    for (int32_t a = 0; a < T; ++a)
      for (const int2& e : lists[s][a]) {
        const int32_t kl = e.y & kLenMask, rlo = (e.y >> kRowLoShift) & 127, rhi = ((e.y >> kRowHiShift) & 127) + 1;
        const int32_t kind = (e.y >> kKindShift) & 3;
        for (int32_t b = e.x / kTile; b <= (e.x + kl - 1) / kTile; ++b) {
          const int32_t klo = std::max(e.x, b * kTile) - b * kTile, khi = std::min(e.x + kl, (b + 1) * kTile) - b * kTile;
          const bool whole = klo == 0 && khi == (int32_t)std::min<int64_t>(kTile, S - (int64_t)b * kTile);
          const bool part = !(kind == kCallFull && whole);
          cols[b].push_back(make_int2(a * kTile + rlo, (rhi - rlo) | (klo << kRowLoShift) | ((khi - 1) << kRowHiShift) |
                                                           (kind << kKindShift) | (part ? kPartialBit : 0)));
        }
      }
    for (int32_t b = 0; b < T; ++b) {
      if (cols[b].empty()) continue;
      std::stable_sort(cols[b].begin(), cols[b].end(), [](const int2& x, const int2& y) { return x.x < y.x; });
      const int32_t kl = (int32_t)std::min<int64_t>(kTile, S - (int64_t)b * kTile);
      st.bitems.push_back(make_int4(b * kTile, kl << kKeyRowsShift, (int32_t)pk.entries.size(),
                                    (int32_t)cols[b].size()));
      pk.entries.insert(pk.entries.end(), cols[b].begin(), cols[b].end());
    }
    std::stable_sort(st.bitems.begin(), st.bitems.end(),
                     [](const int4& x, const int4& y) { return x.w != y.w ? x.w > y.w : x.x < y.x; });
    split_work(st);
  }
  chain_items(pk, T, R, [&](int32_t s, int32_t a) { return (int64_t)lists[s][a].size(); }, qsample);
  pk.sitems.clear();
  for (int32_t a = 0; a < T; ++a) {
    const int32_t beg = (int32_t)pk.entries.size();
    for (int32_t s = 0; s < R; ++s) {
      const int32_t j = ((r - s) % R + R) % R;
      for (const int2& e : lists[s][a]) pk.entries.push_back(make_int2((int32_t)(j * S + e.x), e.y));
    }
    const int32_t cnt = (int32_t)pk.entries.size() - beg;
    if (cnt) pk.sitems.push_back(make_int4(a, kFirst | kLast, beg, cnt));
  }
  order_items(pk.sitems, qsample);
  pk.xitems.clear();
  pk.xtracks.clear();
  pk.xkint.clear();
  pk.yitems.clear();
  pk.xsrc.clear();
  pk.fetch_tiles = pk.fetch_rows = 0;
  layout(p, pk);
  return BSM_OK;
}

}  // namespace bsm

static_assert(bsm::kCallFull == bsm::kRelFull && bsm::kCallCausal == bsm::kRelCausal &&
                  bsm::kCallReverse == bsm::kRelReverse && bsm::kCallPastWindow == bsm::kRelPastWindow &&
                  bsm::kCallFull == BSM_CALL_FULL && bsm::kCallCausal == BSM_CALL_CAUSAL &&
                  bsm::kCallReverse == BSM_CALL_REVERSE && bsm::kCallPastWindow == BSM_CALL_PAST_WINDOW,
              "planner relations and kernel entry relations agree");

struct bsm_dplan {
  int32_t dense = 0;  // forward lists from dense calls (no backward or fetch lists)
  int32_t r = 0, R = 1, tps = 0, window = 0;
  int64_t S = 0, n = 0;
  const int4* tracks = nullptr;
  const int32_t* coord = nullptr;  // per plan row: token index in the caller's order
  const int2* kint = nullptr;
  const int2* entries = nullptr;
  const int4* fitems[64] = {};
  const int2* ffirst[64] = {};
  const int4* citems[64] = {};  // forward items by chain (chain 0 first) and their first entries
  const int2* cfirst[64] = {};
  int64_t nc0[64] = {};         // items of chain 0
  const int4* bitems[64] = {};
  int64_t nf[64] = {}, nb[64] = {}, pairs[64] = {};
  const int4* bwork[64] = {};   // split dK/dV work units
  const int4* breduce[64] = {};
  int64_t nwork[64] = {}, nreduce[64] = {};
  int32_t slots[64] = {};
  int32_t ws_slots = 0;         // max over steps
  const int4* sitems = nullptr;
  const int2* sfirst = nullptr;
  int64_t ns = 0;
  const int4* xitems = nullptr;
  const int2* xfirst = nullptr;
  const int4* xtracks = nullptr;
  const int2* xkint = nullptr;
  int64_t nx = 0, fetch_tiles = 0, fetch_rows = 0;
  const int4* yitems = nullptr;  // the fetched pass's dK/dV column items
  int64_t ny = 0;
  const int32_t* xsrc = nullptr;
};

using namespace bsm;

namespace {

int check_heads(const bsm_heads* h) {
  if (!h) { set_error("heads is NULL"); return BSM_E_INVALID; }
  if (h->hq < 1 || h->hkv < 1 || h->hq % h->hkv) {
    set_error("need hq >= 1, hkv >= 1 and hq % hkv == 0");
    return BSM_E_INVALID;
  }
  if (h->d != kHeadDim) { set_error("only d == 128 is supported"); return BSM_E_UNSUPPORTED; }
  if (!(h->scale > 0.f)) { set_error("scale must be > 0"); return BSM_E_INVALID; }
  return BSM_OK;
}

int32_t heads_per_xcd(int32_t hq) { return hq % 8 == 0 ? hq / 8 : 0; }

// The kernels address a row buffer with 32-bit byte offsets: rows * heads *
// d * 2 bytes must stay below 2^32.
int check_rows(int64_t rows, int32_t heads, const char* what) {
  if ((uint64_t)rows * (uint64_t)heads * kHeadDim * 2u >= (1ull << 32)) {
    set_error(std::string(what) + ": buffers of 4 GiB or more per tensor are not supported");
    return BSM_E_UNSUPPORTED;
  }
  return BSM_OK;
}

const uint16_t* bf(const void* p) { return (const uint16_t*)p; }

// Tensors the kernels move in 16-byte vectors must be 16-byte aligned; the
// fp32 row arrays (m, l, LSE, delta) are read per element and need 4 bytes.
int check_aligned(std::initializer_list<const void*> vec16, std::initializer_list<const void*> row4) {
  for (const void* p : vec16)
    if (p && ((uintptr_t)p & 15u)) {
      set_error("tensor pointer not 16-byte aligned");
      return BSM_E_INVALID;
    }
  for (const void* p : row4)
    if (p && ((uintptr_t)p & 3u)) {
      set_error("row array pointer not 4-byte aligned");
      return BSM_E_INVALID;
    }
  return BSM_OK;
}

}  // namespace

extern "C" {

const char* bsm_last_error(void) { return g_error.c_str(); }

int32_t bsm_version(void) { return 100; }

int bsm_plan_build(const bsm_plan_desc* desc, bsm_plan** out) {
  if (!desc || !out) { set_error("null argument"); return BSM_E_INVALID; }
  *out = nullptr;
  bsm_plan* p = new (std::nothrow) bsm_plan();
  if (!p) { set_error("out of host memory"); return BSM_E_NOMEM; }
  int rc;
  try {
    rc = build_plan(*desc, p->p);
  } catch (const std::bad_alloc&) {
    set_error("out of host memory");
    rc = BSM_E_NOMEM;
  }
  if (rc) {
    delete p;
    return rc;
  }
  *out = p;
  return BSM_OK;
}

void bsm_plan_free(bsm_plan* plan) { delete plan; }

int bsm_plan_get_info(const bsm_plan* plan, bsm_plan_info* out) {
  if (!plan || !out) { set_error("null argument"); return BSM_E_INVALID; }
  const Plan& p = plan->p;
  std::memset(out, 0, sizeof(*out));
  out->n = p.n;
  out->ranks = p.ranks;
  out->block = p.block;
  out->order = p.order;
  out->window = p.window;
  out->shard_tokens = p.shard;
  out->tiles_per_shard = p.tps;
  out->tiles_total = p.ntiles;
  out->busiest_rank = p.busiest;
  out->total_pairs = p.total_pairs;
  out->candidate_pairs = p.candidates;
  out->full_tiles = p.nfull;
  out->partial_tiles = p.npartial;
  out->build_seconds = p.seconds;
  out->interval_keys = p.interval_keys;
  return BSM_OK;
}

int bsm_plan_key_intervals(const bsm_plan* plan, int32_t* lo, int32_t* hi) {
  if (!plan || !lo || !hi) { set_error("null argument"); return BSM_E_INVALID; }
  std::memcpy(lo, plan->p.klo.data(), plan->p.n * sizeof(int32_t));
  std::memcpy(hi, plan->p.khi.data(), plan->p.n * sizeof(int32_t));
  return BSM_OK;
}

int bsm_plan_permutation(const bsm_plan* plan, int32_t* new_to_orig) {
  if (!plan || !new_to_orig) { set_error("null argument"); return BSM_E_INVALID; }
  std::copy(plan->p.perm.begin(), plan->p.perm.end(), new_to_orig);
  return BSM_OK;
}

int bsm_plan_block_cost(const bsm_plan* plan, int64_t* cost, int32_t* owner) {
  if (!plan) { set_error("null plan"); return BSM_E_INVALID; }
  if (cost) std::copy(plan->p.cost.begin(), plan->p.cost.end(), cost);
  if (owner) std::copy(plan->p.owner.begin(), plan->p.owner.end(), owner);
  return BSM_OK;
}

int bsm_plan_step_map(const bsm_plan* plan, int32_t r, int32_t s, uint8_t* map, int64_t* pairs) {
  if (!plan) { set_error("null plan"); return BSM_E_INVALID; }
  if (r < 0 || r >= plan->p.ranks || s < 0 || s >= plan->p.ranks) {
    set_error("rank or step out of range");
    return BSM_E_INVALID;
  }
  const int64_t t = step_map(plan->p, r, s, map);
  if (pairs) *pairs = t;
  return BSM_OK;
}

int bsm_plan_pairs(const bsm_plan* plan, int64_t* pairs) {
  if (!plan || !pairs) { set_error("null argument"); return BSM_E_INVALID; }
  const int32_t R = plan->p.ranks;
  for (int32_t r = 0; r < R; ++r)
    for (int32_t s = 0; s < R; ++s) pairs[(int64_t)r * R + s] = step_map(plan->p, r, s, nullptr);
  return BSM_OK;
}

}  // extern "C"

namespace {
int dplan_bytes(const bsm_plan* plan, int32_t r, bool dense, int64_t* bytes) {
  if (!plan || !bytes) { set_error("null argument"); return BSM_E_INVALID; }
  if (r < 0 || r >= plan->p.ranks) { set_error("rank out of range"); return BSM_E_INVALID; }
  if (plan->p.block != kTile) { set_error("device plans need block == 128"); return BSM_E_UNSUPPORTED; }
  try {
    Packed pk;
    if (dense) {
      const int rc = pack_calls(plan->p, r, pk);
      if (rc) return rc;
    } else {
      pack(plan->p, r, pk);
    }
    *bytes = pk.bytes;
  } catch (const std::bad_alloc&) {
    set_error("out of host memory");
    return BSM_E_NOMEM;
  }
  return BSM_OK;
}

int dplan_upload(const bsm_plan* plan, int32_t r, bool dense, void* dev, int64_t bytes, void* stream,
                 bsm_dplan** out) {
  if (!plan || !dev || !out) { set_error("null argument"); return BSM_E_INVALID; }
  *out = nullptr;
  if (r < 0 || r >= plan->p.ranks) { set_error("rank out of range"); return BSM_E_INVALID; }
  if (plan->p.block != kTile) { set_error("device plans need block == 128"); return BSM_E_UNSUPPORTED; }
  const Plan& p = plan->p;
  try {
    Packed pk;
    if (dense) {
      const int rc = pack_calls(p, r, pk);
      if (rc) return rc;
    } else {
      pack(p, r, pk);
    }
    if (bytes < pk.bytes) {
      set_error("device plan buffer too small: need " + std::to_string(pk.bytes) + " bytes");
      return BSM_E_NOMEM;
    }
    std::vector<char> img(pk.bytes, 0);
    std::memcpy(img.data() + pk.off_tracks, pk.tracks.data(), pk.tracks.size() * sizeof(int4));
    std::memcpy(img.data() + pk.off_coord, pk.coord.data(), pk.coord.size() * sizeof(int32_t));
    std::memcpy(img.data() + pk.off_kint, pk.kint.data(), pk.kint.size() * sizeof(int2));
    for (int32_t s = 0; s < p.ranks; ++s) {
      std::memcpy(img.data() + pk.off_f[s], pk.steps[s].fitems.data(), pk.steps[s].fitems.size() * sizeof(int4));
      int2* ff = (int2*)(img.data() + pk.off_ff[s]);
      for (size_t i = 0; i < pk.steps[s].fitems.size(); ++i) ff[i] = pk.entries[pk.steps[s].fitems[i].z];
      std::memcpy(img.data() + pk.off_c[s], pk.steps[s].citems.data(), pk.steps[s].citems.size() * sizeof(int4));
      int2* cf = (int2*)(img.data() + pk.off_cf[s]);
      for (size_t i = 0; i < pk.steps[s].citems.size(); ++i) cf[i] = pk.entries[pk.steps[s].citems[i].z];
      std::memcpy(img.data() + pk.off_b[s], pk.steps[s].bitems.data(), pk.steps[s].bitems.size() * sizeof(int4));
      std::memcpy(img.data() + pk.off_w[s], pk.steps[s].bwork.data(), pk.steps[s].bwork.size() * sizeof(int4));
      std::memcpy(img.data() + pk.off_r[s], pk.steps[s].breduce.data(), pk.steps[s].breduce.size() * sizeof(int4));
    }
    std::memcpy(img.data() + pk.off_s, pk.sitems.data(), pk.sitems.size() * sizeof(int4));
    int2* sf = (int2*)(img.data() + pk.off_sf);
    for (size_t i = 0; i < pk.sitems.size(); ++i) sf[i] = pk.entries[pk.sitems[i].z];
    std::memcpy(img.data() + pk.off_x, pk.xitems.data(), pk.xitems.size() * sizeof(int4));
    int2* xf = (int2*)(img.data() + pk.off_xf);
    for (size_t i = 0; i < pk.xitems.size(); ++i) xf[i] = pk.entries[pk.xitems[i].z];
    std::memcpy(img.data() + pk.off_xtracks, pk.xtracks.data(), pk.xtracks.size() * sizeof(int4));
    std::memcpy(img.data() + pk.off_xkint, pk.xkint.data(), pk.xkint.size() * sizeof(int2));
    std::memcpy(img.data() + pk.off_y, pk.yitems.data(), pk.yitems.size() * sizeof(int4));
    std::memcpy(img.data() + pk.off_xsrc, pk.xsrc.data(), pk.xsrc.size() * sizeof(int32_t));
    std::memcpy(img.data() + pk.off_entries, pk.entries.data(), pk.entries.size() * sizeof(int2));
    hipStream_t st = (hipStream_t)stream;
    int rc = hip_status(hipMemcpyAsync(dev, img.data(), pk.bytes, hipMemcpyHostToDevice, st),
                        "plan upload", st);
    if (rc) return rc;
    rc = hip_status(hipStreamSynchronize(st), "plan upload sync", st);
    if (rc) return rc;
    bsm_dplan* d = new bsm_dplan();
    char* base = (char*)dev;
    d->dense = dense ? 1 : 0;
    d->r = r;
    d->R = p.ranks;
    d->tps = p.tps;
    d->window = p.window;
    d->S = p.shard;
    d->n = p.n;
    d->tracks = (const int4*)(base + pk.off_tracks);
    d->coord = (const int32_t*)(base + pk.off_coord);
    d->kint = (const int2*)(base + pk.off_kint);
    d->entries = (const int2*)(base + pk.off_entries);
    for (int32_t s = 0; s < p.ranks; ++s) {
      d->fitems[s] = (const int4*)(base + pk.off_f[s]);
      d->ffirst[s] = (const int2*)(base + pk.off_ff[s]);
      d->citems[s] = (const int4*)(base + pk.off_c[s]);
      d->cfirst[s] = (const int2*)(base + pk.off_cf[s]);
      d->nc0[s] = pk.steps[s].nchain0;
      d->bitems[s] = (const int4*)(base + pk.off_b[s]);
      d->nf[s] = (int64_t)pk.steps[s].fitems.size();
      d->nb[s] = (int64_t)pk.steps[s].bitems.size();
      d->pairs[s] = pk.steps[s].pairs;
      d->bwork[s] = (const int4*)(base + pk.off_w[s]);
      d->breduce[s] = (const int4*)(base + pk.off_r[s]);
      d->nwork[s] = (int64_t)pk.steps[s].bwork.size();
      d->nreduce[s] = (int64_t)pk.steps[s].breduce.size();
      d->slots[s] = pk.steps[s].slots;
      d->ws_slots = std::max(d->ws_slots, pk.steps[s].slots);
    }
    d->sitems = (const int4*)(base + pk.off_s);
    d->sfirst = (const int2*)(base + pk.off_sf);
    d->ns = (int64_t)pk.sitems.size();
    d->xitems = (const int4*)(base + pk.off_x);
    d->xfirst = (const int2*)(base + pk.off_xf);
    d->xtracks = (const int4*)(base + pk.off_xtracks);
    d->xkint = (const int2*)(base + pk.off_xkint);
    d->nx = (int64_t)pk.xitems.size();
    d->fetch_tiles = pk.fetch_tiles;
    d->fetch_rows = pk.fetch_rows;
    d->yitems = (const int4*)(base + pk.off_y);
    d->ny = (int64_t)pk.yitems.size();
    d->xsrc = (const int32_t*)(base + pk.off_xsrc);
    *out = d;
  } catch (const std::bad_alloc&) {
    set_error("out of host memory");
    return BSM_E_NOMEM;
  }
  return BSM_OK;
}
}  // namespace

extern "C" {

int bsm_dplan_bytes(const bsm_plan* plan, int32_t r, int64_t* bytes) {
  return dplan_bytes(plan, r, false, bytes);
}

int bsm_dplan_upload(const bsm_plan* plan, int32_t r, void* dev, int64_t bytes, void* stream,
                     bsm_dplan** out) {
  return dplan_upload(plan, r, false, dev, bytes, stream, out);
}

int bsm_dplan_calls_bytes(const bsm_plan* plan, int32_t r, int64_t* bytes) {
  return dplan_bytes(plan, r, true, bytes);
}

int bsm_dplan_calls_upload(const bsm_plan* plan, int32_t r, void* dev, int64_t bytes, void* stream,
                           bsm_dplan** out) {
  return dplan_upload(plan, r, true, dev, bytes, stream, out);
}

int bsm_plan_dense_calls(const bsm_plan* plan, int32_t r, int32_t s, bsm_call* calls, int64_t capacity,
                         int64_t* count) {
  if (!plan || !count) { set_error("null argument"); return BSM_E_INVALID; }
  if (r < 0 || r >= plan->p.ranks || s < 0 || s >= plan->p.ranks) {
    set_error("rank or step out of range");
    return BSM_E_INVALID;
  }
  try {
    std::vector<Call> v;
    const int rc = dense_calls(plan->p, r, s, v);
    if (rc) return rc;
    *count = (int64_t)v.size();
    if (!calls) return BSM_OK;
    if (capacity < (int64_t)v.size()) {
      set_error("call buffer too small: need " + std::to_string(v.size()) + " calls");
      return BSM_E_NOMEM;
    }
    for (size_t i = 0; i < v.size(); ++i) calls[i] = bsm_call{v[i].q0, v[i].qn, v[i].k0, v[i].kn, v[i].kind};
  } catch (const std::bad_alloc&) {
    set_error("out of host memory");
    return BSM_E_NOMEM;
  }
  return BSM_OK;
}

void bsm_dplan_free(bsm_dplan* dplan) { delete dplan; }

int bsm_dplan_get_info(const bsm_dplan* d, bsm_dplan_info* out) {
  if (!d || !out) { set_error("null argument"); return BSM_E_INVALID; }
  std::memset(out, 0, sizeof(*out));
  out->rank = d->r;
  out->ranks = d->R;
  out->shard_tokens = d->S;
  out->tiles_per_shard = d->tps;
  out->window = d->window;
  for (int32_t s = 0; s < d->R; ++s) {
    out->fwd_items[s] = d->nf[s];
    out->fwd_chain0_items[s] = d->nc0[s];
    out->bwd_items[s] = d->nb[s];
    out->step_pairs[s] = d->pairs[s];
  }
  out->single_items = d->ns;
  out->fetch_tiles = d->fetch_tiles;
  out->fetch_rows = d->fetch_rows;
  out->dense_calls = d->dense;
  out->bwd_workspace_slots = d->ws_slots;
  return BSM_OK;
}

}  // extern "C"

namespace {
// One ring step's launch over `n` forward items (with their first list
// entries) of step s: all of them (bsm_fwd_step) or one chain's.
int fwd_step_items(const bsm_dplan* d, int32_t s, const bsm_heads* heads, const void* q, const void* k,
                   const void* v, float* o_acc, float* m, float* l, void* o, float* lse, int32_t flags,
                   void* stream, int32_t chain) {
  if (!d) { set_error("null device plan"); return BSM_E_INVALID; }
  int rc = check_heads(heads);
  if (rc) return rc;
  if (s < 0 || s >= d->R) { set_error("step out of range"); return BSM_E_INVALID; }
  const bool keep = (flags & BSM_FWD_KEEP_STATE) != 0;
  if (!q || !k || !v || !o_acc || !m || !l || (!keep && (!o || !lse))) {
    set_error("null tensor pointer");
    return BSM_E_INVALID;
  }
  if ((rc = check_rows(d->S, heads->hq, "q")) || (rc = check_rows(d->S, heads->hkv, "k/v"))) return rc;
  if ((rc = check_aligned({q, k, v, o_acc, o}, {m, l, lse}))) return rc;
  if (chain < -1 || chain > 1) { set_error("chain must be 0 or 1"); return BSM_E_INVALID; }
  const int64_t i0 = chain == 1 ? d->nc0[s] : 0, i1 = chain == 0 ? d->nc0[s] : d->nf[s];
  if (i1 <= i0) return BSM_OK;
  const int32_t j = ((d->r - s) % d->R + d->R) % d->R;
  FwdArgs a{};
  a.items = chain < 0 ? d->fitems[s] : d->citems[s] + i0;
  a.first = chain < 0 ? d->ffirst[s] : d->cfirst[s] + i0;
  a.entries = d->entries;
  a.nitems = (int32_t)(i1 - i0);
  a.hq = heads->hq;
  a.hkv = heads->hkv;
  a.heads_per_xcd = heads_per_xcd(heads->hq);
  a.q = bf(q);
  a.k = bf(k);
  a.v = bf(v);
  a.qtracks = d->tracks + (int64_t)d->r * d->S;
  a.qcoord = d->coord + (int64_t)d->r * d->S;
  a.ktracks = d->tracks + (int64_t)j * d->S;
  a.kint = d->kint + (int64_t)j * d->S;
  a.rows = d->S;
  a.oacc = o_acc;
  a.m = m;
  a.l = l;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.scale_log2 = heads->scale * 1.44269504088896340736f;
  a.window = d->window;
  a.keep_state = keep ? 1 : 0;
  a.step_only = (flags & BSM_FWD_STEP_ONLY) != 0 ? 1 : 0;
  a.dense = d->dense;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_fwd(a, st), "forward step launch", st);
}
}  // namespace

extern "C" {

int bsm_fwd_step(const bsm_dplan* d, int32_t s, const bsm_heads* heads, const void* q,
                 const void* k, const void* v, float* o_acc, float* m, float* l, void* o,
                 float* lse, int32_t flags, void* stream) {
  return fwd_step_items(d, s, heads, q, k, v, o_acc, m, l, o, lse, flags, stream, -1);
}

int bsm_fwd_step_chain(const bsm_dplan* d, int32_t s, int32_t chain, const bsm_heads* heads, const void* q,
                       const void* k, const void* v, float* o_acc, float* m, float* l, void* o, float* lse,
                       int32_t flags, void* stream) {
  if (chain != 0 && chain != 1) { set_error("chain must be 0 or 1"); return BSM_E_INVALID; }
  return fwd_step_items(d, s, heads, q, k, v, o_acc, m, l, o, lse, flags, stream, chain);
}

namespace {
// One pass over merged lists (`fetched`: the sparse-fetch lists over the
// compact buffer; otherwise the single-pass lists over all shards).
int fwd_pass(const bsm_dplan* d, bool fetched, const bsm_heads* heads, const void* q, const void* k_all,
             const void* v_all, float* o_acc, float* m, float* l, void* o, float* lse, int32_t flags,
             void* stream) {
  if (!d) { set_error("null device plan"); return BSM_E_INVALID; }
  int rc = check_heads(heads);
  if (rc) return rc;
  const bool keep = (flags & BSM_FWD_KEEP_STATE) != 0;
  if (!q || !k_all || !v_all || (keep && (!o_acc || !m || !l)) || (!keep && (!o || !lse))) {
    set_error("null tensor pointer");
    return BSM_E_INVALID;
  }
  if (fetched && d->dense) {
    set_error("a dense-call device plan has no sparse-fetch lists");
    return BSM_E_UNSUPPORTED;
  }
  const int64_t krows = fetched ? d->fetch_rows : (int64_t)d->S * d->R;
  if ((rc = check_rows(d->S, heads->hq, "q")) || (rc = check_rows(krows, heads->hkv, "keys/values")))
    return rc;
  if ((rc = check_aligned({q, k_all, v_all, o_acc, o}, {m, l, lse}))) return rc;
  const int64_t nitems = fetched ? d->nx : d->ns;
  if (nitems == 0) return BSM_OK;
  FwdArgs a{};
  a.items = fetched ? d->xitems : d->sitems;
  a.first = fetched ? d->xfirst : d->sfirst;
  a.entries = d->entries;
  a.nitems = (int32_t)nitems;
  a.hq = heads->hq;
  a.hkv = heads->hkv;
  a.heads_per_xcd = heads_per_xcd(heads->hq);
  a.q = bf(q);
  a.k = bf(k_all);
  a.v = bf(v_all);
  a.qtracks = d->tracks + (int64_t)d->r * d->S;
  a.qcoord = d->coord + (int64_t)d->r * d->S;
  a.ktracks = fetched ? d->xtracks : d->tracks;
  a.kint = fetched ? d->xkint : d->kint;
  a.rows = d->S;
  a.oacc = o_acc;
  a.m = m;
  a.l = l;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.scale_log2 = heads->scale * 1.44269504088896340736f;
  a.window = d->window;
  a.keep_state = keep ? 1 : 0;
  a.step_only = (flags & BSM_FWD_STEP_ONLY) != 0 ? 1 : 0;
  a.dense = d->dense;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_fwd(a, st), fetched ? "forward fetched launch" : "forward single launch", st);
}
}  // namespace

int bsm_fwd_single(const bsm_dplan* d, const bsm_heads* heads, const void* q, const void* k_all,
                   const void* v_all, float* o_acc, float* m, float* l, void* o, float* lse,
                   int32_t flags, void* stream) {
  return fwd_pass(d, false, heads, q, k_all, v_all, o_acc, m, l, o, lse, flags, stream);
}

int bsm_fwd_fetched(const bsm_dplan* d, const bsm_heads* heads, const void* q, const void* k_fetch,
                    const void* v_fetch, float* o_acc, float* m, float* l, void* o, float* lse,
                    int32_t flags, void* stream) {
  return fwd_pass(d, true, heads, q, k_fetch, v_fetch, o_acc, m, l, o, lse, flags, stream);
}

int bsm_plan_chunk_order(const bsm_plan* plan, int32_t min_chunks, int32_t max_chunks, double tau,
                         int32_t swaps, int32_t* block_perm, bsm_chunk_info* out) {
  if (!plan || !block_perm || !out) { set_error("null argument"); return BSM_E_INVALID; }
  ChunkResult res;
  const int rc = chunk_order(plan->p, min_chunks, max_chunks, tau, swaps, block_perm, res);
  if (rc) return rc;
  out->chunks_per_rank = res.chunks_per_rank;
  out->strategy = res.strategy;
  out->cost = res.cost;
  out->step_max_sum = res.step_max_sum;
  out->range_term = res.range_term;
  return BSM_OK;
}

int bsm_vision_group_order(int64_t n, const int32_t* sample, const int32_t* seg, int32_t* new_to_orig) {
  try {
    return vision_group_order(n, sample, seg, new_to_orig);
  } catch (const std::bad_alloc&) {
    set_error("out of host memory");
    return BSM_E_NOMEM;
  }
}

int bsm_plan_fetch_set(const bsm_plan* plan, int32_t r, uint8_t* needed, int64_t* tiles) {
  if (!plan || !needed) { set_error("null argument"); return BSM_E_INVALID; }
  if (r < 0 || r >= plan->p.ranks) { set_error("rank out of range"); return BSM_E_INVALID; }
  const int64_t c = fetch_set(plan->p, r, needed);
  if (tiles) *tiles = c;
  return BSM_OK;
}

int bsm_fwd_merge_bf16(const bsm_heads* heads, int64_t rows, void* o_run, float* lse_run, const void* o_s,
                       const float* lse_s, void* stream) {
  int rc = check_heads(heads);
  if (rc) return rc;
  if (rows < 1) { set_error("rows must be >= 1"); return BSM_E_INVALID; }
  if (!o_run || !lse_run || !o_s || !lse_s) { set_error("null tensor pointer"); return BSM_E_INVALID; }
  if ((rc = check_aligned({o_run, o_s}, {lse_run, lse_s}))) return rc;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_merge_bf16(rows, heads->hq, (uint16_t*)o_run, lse_run, bf(o_s), lse_s, st),
                    "bf16 merge launch", st);
}

int bsm_fwd_merge_fp32(const bsm_heads* heads, int64_t rows, float* o_run, float* lse_run, const float* acc_s,
                       const float* m_s, const float* l_s, void* o_bf16, void* stream) {
  int rc = check_heads(heads);
  if (rc) return rc;
  if (rows < 1) { set_error("rows must be >= 1"); return BSM_E_INVALID; }
  if (!o_run || !lse_run || !acc_s || !m_s || !l_s) { set_error("null tensor pointer"); return BSM_E_INVALID; }
  if ((rc = check_aligned({o_run, acc_s, o_bf16}, {lse_run, m_s, l_s}))) return rc;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_merge_fp32(rows, heads->hq, o_run, lse_run, acc_s, m_s, l_s, (uint16_t*)o_bf16, st),
                    "fp32 merge launch", st);
}

int bsm_state_unpack(const bsm_heads* heads, int64_t rows, const float* o_acc, float* out, void* stream) {
  int rc = check_heads(heads);
  if (rc) return rc;
  if (rows < 1) { set_error("rows must be >= 1"); return BSM_E_INVALID; }
  if (!o_acc || !out) { set_error("null tensor pointer"); return BSM_E_INVALID; }
  if ((rc = check_aligned({o_acc, out}, {}))) return rc;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_state_unpack(rows, heads->hq, o_acc, out, st), "state unpack launch", st);
}

int bsm_bwd_prep(const bsm_heads* heads, int64_t rows, const void* o, const void* dout,
                 float* delta, void* stream) {
  int rc = check_heads(heads);
  if (rc) return rc;
  if (rows < 1) { set_error("rows must be >= 1"); return BSM_E_INVALID; }
  if (!o || !dout || !delta) { set_error("null tensor pointer"); return BSM_E_INVALID; }
  if ((rc = check_aligned({o, dout}, {delta}))) return rc;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_bwd_prep(rows, heads->hq, bf(o), bf(dout), delta, st), "bwd prep launch", st);
}

}  // extern "C"

namespace {
// Workgroups a launch should have to keep every CU busy past its longest
// item: twice the CU count of the current device.
int64_t busy_blocks() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  return 2 * (int64_t)cus;
}

// Workspace bytes step s needs when its dK/dV work is split: the split is
// taken when the plan cut long column lists at that step and the step has
// fewer (key tile, kv head) units than twice the CUs; 0 otherwise.
int64_t split_bytes(const bsm_dplan* d, int32_t s, const bsm_heads* heads) {
  if (d->nreduce[s] == 0 || d->nb[s] * heads->hkv >= busy_blocks()) return 0;
  return (int64_t)d->slots[s] * heads->hkv * 2 * kTile * kHeadDim * (int64_t)sizeof(float);
}

int bwd_step(const bsm_dplan* d, int32_t s, const bsm_heads* heads, const void* q, const void* k, const void* v,
             const void* dout, const float* lse, const float* delta, float* dq_acc, float* dk, float* dv,
             void* workspace, int64_t workspace_bytes, void* stream, void* kv_stream) {
  if (!d) { set_error("null device plan"); return BSM_E_INVALID; }
  int rc = check_heads(heads);
  if (rc) return rc;
  if (s < 0 || s >= d->R) { set_error("step out of range"); return BSM_E_INVALID; }
  if (!q || !k || !v || !dout || !lse || !delta || !dq_acc || !dk || !dv) {
    set_error("null tensor pointer");
    return BSM_E_INVALID;
  }
  if ((rc = check_rows(d->S, heads->hq, "q/dout")) || (rc = check_rows(d->S, heads->hkv, "k/v"))) return rc;
  if ((rc = check_aligned({q, k, v, dout, dq_acc, dk, dv, workspace}, {lse, delta}))) return rc;
  // split the dK/dV work when a workspace is given and the launch would
  // otherwise leave CUs waiting on its longest column lists
  const int64_t need = workspace ? split_bytes(d, s, heads) : 0;
  const bool split = need > 0;
  if (split) {
    if (workspace_bytes < need) {
      set_error("backward workspace too small: need " + std::to_string(need) + " bytes");
      return BSM_E_INVALID;
    }
  }
  const int32_t j = ((d->r - s) % d->R + d->R) % d->R;
  BwdArgs a{};
  a.entries = d->entries;
  a.hq = heads->hq;
  a.hkv = heads->hkv;
  a.heads_per_xcd = heads_per_xcd(heads->hq);
  a.q = bf(q);
  a.k = bf(k);
  a.v = bf(v);
  a.dout = bf(dout);
  a.lse = lse;
  a.delta = delta;
  a.qtracks = d->tracks + (int64_t)d->r * d->S;
  a.qcoord = d->coord + (int64_t)d->r * d->S;
  a.ktracks = d->tracks + (int64_t)j * d->S;
  a.kint = d->kint + (int64_t)j * d->S;
  a.dense = d->dense;
  a.rows = d->S;
  a.krows = d->S;
  a.dq = dq_acc;
  a.dk = dk;
  a.dv = dv;
  a.scale = heads->scale;
  a.scale_log2 = heads->scale * 1.44269504088896340736f;
  a.window = d->window;
  hipStream_t st = (hipStream_t)stream;
  if (d->nf[s]) {
    a.items = d->fitems[s];
    a.nitems = (int32_t)d->nf[s];
    rc = hip_status(launch_bwd_dq(a, st), "bwd dq launch", st);
    if (rc) return rc;
  }
  st = (hipStream_t)kv_stream;
  if (d->nb[s]) {
    a.items = d->bitems[s];
    a.heads_per_xcd = heads->hkv % 8 == 0 ? heads->hkv / 8 : 0;
    if (split) {
      a.work = d->bwork[s];
      a.nitems = (int32_t)d->nwork[s];
      a.ws = (float*)workspace;
      a.reduce = d->breduce[s];
      a.nreduce = (int32_t)d->nreduce[s];
      rc = hip_status(launch_bwd_dkdv(a, st), "bwd dkdv launch", st);
      if (rc) return rc;
      rc = hip_status(launch_bwd_reduce(a, st), "bwd reduce launch", st);
    } else {
      a.nitems = (int32_t)d->nb[s];
      rc = hip_status(launch_bwd_dkdv(a, st), "bwd dkdv launch", st);
    }
  }
  return rc;
}
// Scratch of bsm_bwd_step_noalloc: the split dK/dV partial sums of a step
// go here instead of into a caller workspace.  Every device the library runs
// on holds its own copy from the module load until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: kernels
// get the address hipGetSymbolAddress returns for the current device.
constexpr int64_t kScratchBytes = 64ll << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up on the first call on that
// device (with the device current) and kept.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(std::string("hipGetDevice: ") + hipGetErrorString(e));
    return BSM_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device index beyond the scratch table");
    return BSM_E_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error(std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
      return BSM_E_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BSM_OK;
}
}  // namespace

extern "C" {

int bsm_bwd_step_noalloc(const bsm_dplan* d, int32_t s, const bsm_heads* heads, const void* q, const void* k,
                         const void* v, const void* dout, const float* lse, const float* delta, float* dq_acc,
                         float* dk, float* dv, void* stream) {
  if (!d) { set_error("null device plan"); return BSM_E_INVALID; }
  int rc = check_heads(heads);
  if (rc) return rc;
  if (s < 0 || s >= d->R) { set_error("step out of range"); return BSM_E_INVALID; }
  const int64_t need = split_bytes(d, s, heads);
  if (need > kScratchBytes) {
    set_error("bsm_bwd_step_noalloc: step " + std::to_string(s) + " needs " + std::to_string(need) +
              " bytes of split-work scratch, the static scratch holds " + std::to_string(kScratchBytes) +
              "; use bsm_bwd_step_ws with a caller workspace");
    return BSM_E_UNSUPPORTED;
  }
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return bwd_step(d, s, heads, q, k, v, dout, lse, delta, dq_acc, dk, dv, ws, kScratchBytes, stream, stream);
}

int bsm_bwd_step(const bsm_dplan* d, int32_t s, const bsm_heads* heads, const void* q,
                 const void* k, const void* v, const void* dout, const float* lse,
                 const float* delta, float* dq_acc, float* dk, float* dv, void* stream) {
  return bwd_step(d, s, heads, q, k, v, dout, lse, delta, dq_acc, dk, dv, nullptr, 0, stream, stream);
}

int bsm_bwd_step_ws(const bsm_dplan* d, int32_t s, const bsm_heads* heads, const void* q, const void* k,
                    const void* v, const void* dout, const float* lse, const float* delta, float* dq_acc,
                    float* dk, float* dv, void* workspace, int64_t workspace_bytes, void* stream) {
  return bwd_step(d, s, heads, q, k, v, dout, lse, delta, dq_acc, dk, dv, workspace, workspace_bytes, stream,
                  stream);
}

int bsm_bwd_step_streams(const bsm_dplan* d, int32_t s, const bsm_heads* heads, const void* q, const void* k,
                         const void* v, const void* dout, const float* lse, const float* delta, float* dq_acc,
                         float* dk, float* dv, void* workspace, int64_t workspace_bytes, void* dq_stream,
                         void* kv_stream) {
  return bwd_step(d, s, heads, q, k, v, dout, lse, delta, dq_acc, dk, dv, workspace, workspace_bytes, dq_stream,
                  kv_stream);
}

int bsm_bwd_fetched(const bsm_dplan* d, const bsm_heads* heads, const void* q, const void* k_fetch,
                    const void* v_fetch, const void* dout, const float* lse, const float* delta, float* dq,
                    float* dk_fetch, float* dv_fetch, void* stream) {
  if (!d) { set_error("null device plan"); return BSM_E_INVALID; }
  int rc = check_heads(heads);
  if (rc) return rc;
  if (d->dense) {
    set_error("a dense-call device plan has no sparse-fetch lists");
    return BSM_E_UNSUPPORTED;
  }
  if (!q || !k_fetch || !v_fetch || !dout || !lse || !delta || !dq || !dk_fetch || !dv_fetch) {
    set_error("null tensor pointer");
    return BSM_E_INVALID;
  }
  if ((rc = check_rows(d->S, heads->hq, "q/dout")) || (rc = check_rows(d->fetch_rows, heads->hkv, "k/v fetched")))
    return rc;
  if ((rc = check_aligned({q, k_fetch, v_fetch, dout, dq, dk_fetch, dv_fetch}, {lse, delta}))) return rc;
  BwdArgs a{};
  a.entries = d->entries;
  a.hq = heads->hq;
  a.hkv = heads->hkv;
  a.q = bf(q);
  a.k = bf(k_fetch);
  a.v = bf(v_fetch);
  a.dout = bf(dout);
  a.lse = lse;
  a.delta = delta;
  a.qtracks = d->tracks + (int64_t)d->r * d->S;
  a.qcoord = d->coord + (int64_t)d->r * d->S;
  a.ktracks = d->xtracks;
  a.kint = d->xkint;
  a.dense = 0;
  a.rows = d->S;
  a.krows = d->fetch_rows;
  a.dq = dq;
  a.dk = dk_fetch;
  a.dv = dv_fetch;
  a.scale = heads->scale;
  a.scale_log2 = heads->scale * 1.44269504088896340736f;
  a.window = d->window;
  hipStream_t st = (hipStream_t)stream;
  if (d->nx) {
    a.items = d->xitems;
    a.nitems = (int32_t)d->nx;
    a.heads_per_xcd = heads_per_xcd(heads->hq);
    if ((rc = hip_status(launch_bwd_dq(a, st), "bwd fetched dq launch", st))) return rc;
  }
  if (d->ny) {
    a.items = d->yitems;
    a.nitems = (int32_t)d->ny;
    a.heads_per_xcd = heads->hkv % 8 == 0 ? heads->hkv / 8 : 0;
    if ((rc = hip_status(launch_bwd_dkdv(a, st), "bwd fetched dkdv launch", st))) return rc;
  }
  return BSM_OK;
}

int bsm_fetched_accumulate(const bsm_dplan* d, const bsm_heads* heads, const float* dk_fetch,
                           const float* dv_fetch, float* dk_all, float* dv_all, void* stream) {
  if (!d) { set_error("null device plan"); return BSM_E_INVALID; }
  int rc = check_heads(heads);
  if (rc) return rc;
  if (d->dense) {
    set_error("a dense-call device plan has no sparse-fetch lists");
    return BSM_E_UNSUPPORTED;
  }
  if (!dk_fetch || !dv_fetch || !dk_all || !dv_all) {
    set_error("null tensor pointer");
    return BSM_E_INVALID;
  }
  if ((rc = check_aligned({dk_fetch, dv_fetch, dk_all, dv_all}, {}))) return rc;
  FetchAccArgs a{};
  a.src = d->xsrc;
  a.rows = d->fetch_rows;
  a.hkv = heads->hkv;
  a.dk_fetch = dk_fetch;
  a.dv_fetch = dv_fetch;
  a.dk = dk_all;
  a.dv = dv_all;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_fetch_accumulate(a, st), "fetched accumulate launch", st);
}

}  // extern "C"
