// Host planner: metadata tracks -> exact tile classes, pair counts, PTRR order.
//
// MARBLE ("exact sequence parallelism for packed multimodal masks"):
//   section 01, mask_mod code block   - the legality predicate over the tracks
//   section 03, "Block classification" - full / empty / partial tile pairs,
//                                         classified from per-tile summaries
//   section 03, "PTRR"                 - sort blocks by cost, deal in rounds of
//                                         R, reverse every other round, keep
//                                         each rank's blocks in sequence order
//   section 04, "Planning cost"        - built once per batch on CPU threads
//
// Key intervals: for each key the planner also derives the set of queries it
// is legal for from the track structure (its causal window, the tokens of its
// seg id, the tokens of its noise id, its sample); when that set is one range
// of token indices (in the caller's order) the kernels test partial tiles
// with one unsigned compare per pair.
//
// Classification is exact: a tile pair is FULL when every valid token pair is
// legal, EMPTY when none is, PARTIAL otherwise.  Per-tile summaries (min/max of
// every track) decide a pair only when they prove it; every other candidate
// pair is counted token pair by token pair.  Candidate key tiles of a query
// tile are the tiles whose sample-id range meets the query tile's, which is a
// contiguous run of tiles because samples are contiguous runs in the original
// order and tiles are contiguous pieces of it.
//
// Positions need not rise with the index: a layout transform (MARBLE section
// 04, "Layout transforms") may permute tokens, each carrying its original
// position.  Only the dense calls need rising positions.

#include "planner.hpp"

#include <algorithm>
#include <atomic>
#include <chrono>
#include <numeric>
#include <thread>
#include <unordered_map>
#include <cstring>
#include <utility>

namespace bsm {

namespace {

struct Summary {
  int32_t smin, smax, gmin, gmax, nmin, nmax, pmin, pmax;
};

Summary summarize(const Plan& p, int64_t a, int64_t b) {
  Summary s{p.sample[a], p.sample[b - 1], INT32_MAX, INT32_MIN, INT32_MAX, INT32_MIN, INT32_MAX, INT32_MIN};
  for (int64_t i = a; i < b; ++i) {
    s.gmin = std::min(s.gmin, p.seg[i]);
    s.gmax = std::max(s.gmax, p.seg[i]);
    s.nmin = std::min(s.nmin, p.noise[i]);
    s.nmax = std::max(s.nmax, p.noise[i]);
    s.pmin = std::min(s.pmin, p.pos[i]);
    s.pmax = std::max(s.pmax, p.pos[i]);
  }
  return s;
}

// Exact number of legal pairs between query tokens [qa, qb) and key tokens [ka, kb).
int64_t count_pairs(const Plan& p, int64_t qa, int64_t qb, int64_t ka, int64_t kb) {
  const int32_t* ks = p.sample.data() + ka;
  const int32_t* kg = p.seg.data() + ka;
  const int32_t* kn = p.noise.data() + ka;
  const int32_t* kp = p.pos.data() + ka;
  const int64_t nk = kb - ka;
  const int32_t w = p.window;
  int64_t total = 0;
  for (int64_t q = qa; q < qb; ++q) {
    const int32_t sq = p.sample[q], gq = p.seg[q], nq = p.noise[q], pq = p.pos[q];
    int32_t c = 0;
    for (int64_t j = 0; j < nk; ++j) {
      const int32_t d = pq - kp[j];  // positions lie in [0, 2^31): no overflow
      const bool causal = (d >= 0) & (d < w);
      const bool span = (gq == kg[j]) & (kg[j] >= 0);
      const bool keep = (kn[j] < 0) | (nq == kn[j]);
      c += (int32_t)((causal | span) & keep & (sq == ks[j]));
    }
    total += c;
  }
  return total;
}

// Summary-only proof: +1 provably FULL, -1 provably EMPTY, 0 undecided.
int prove(const Summary& q, const Summary& k, int32_t w) {
  if (q.smax < k.smin || k.smax < q.smin) return -1;
  // every key is one noise span that no query belongs to
  if (k.nmin == k.nmax && k.nmin >= 0 && (q.nmax < k.nmin || q.nmin > k.nmin)) return -1;
  const int64_t dmax = (int64_t)q.pmax - k.pmin;  // largest pos_q - pos_k
  const int64_t dmin = (int64_t)q.pmin - k.pmax;  // smallest
  const bool causal_none = dmax < 0 || dmin >= w;
  const bool span_none = q.gmax < 0 || k.gmax < 0 || q.gmax < k.gmin || k.gmax < q.gmin;
  if (causal_none && span_none) return -1;
  const bool one_sample = q.smin == q.smax && k.smin == k.smax && q.smin == k.smin;
  const bool keep_all = k.nmax < 0 ||
                        (q.nmin == q.nmax && k.nmin == k.nmax && q.nmin == k.nmin);
  const bool causal_all = dmin >= 0 && dmax < w;
  const bool span_all = q.gmin == q.gmax && k.gmin == k.gmax && q.gmin == k.gmin && k.gmin >= 0;
  if (one_sample && keep_all && (causal_all || span_all)) return 1;
  return 0;
}

int validate(const bsm_plan_desc& d) {
  if (d.n < 1 || d.n > (int64_t(1) << 30)) { set_error("n must be in [1, 2^30]"); return BSM_E_INVALID; }
  if (!d.sample || !d.seg || !d.noise || !d.pos) { set_error("null track pointer"); return BSM_E_INVALID; }
  if (d.window < 1) { set_error("window must be >= 1"); return BSM_E_INVALID; }
  if (d.ranks < 1 || d.ranks > 64) { set_error("ranks must be in [1, 64]"); return BSM_E_INVALID; }
  if (d.block < 1 || d.block > (1 << 20)) { set_error("block must be in [1, 2^20]"); return BSM_E_INVALID; }
  if (d.order == BSM_ORDER_CONTIGUOUS) {
    if (d.n % d.ranks) { set_error("contiguous order needs n % ranks == 0"); return BSM_E_INVALID; }
  } else if (d.order == BSM_ORDER_PTRR || d.order == BSM_ORDER_EXPLICIT) {
    if (d.n % ((int64_t)d.block * d.ranks)) {
      set_error("block orders need n % (block * ranks) == 0");
      return BSM_E_INVALID;
    }
    if (d.order == BSM_ORDER_EXPLICIT && !d.explicit_block_perm) {
      set_error("explicit order needs explicit_block_perm");
      return BSM_E_INVALID;
    }
  } else {
    set_error("unknown order");
    return BSM_E_INVALID;
  }
  for (int64_t i = 0; i < d.n; ++i) {
    // The kernels give rows and keys past a ragged tile's valid rows sample id
    // -1, which must equal no real sample.
    if (d.sample[i] < 0) { set_error("sample ids must be >= 0"); return BSM_E_INVALID; }
    if (d.seg[i] < -1 || d.noise[i] < -1) { set_error("seg and noise ids must be >= -1"); return BSM_E_INVALID; }
    if (d.pos[i] < 0) { set_error("pos must be >= 0"); return BSM_E_INVALID; }
    if (i > 0 && d.sample[i] < d.sample[i - 1]) {
      set_error("samples must be contiguous runs with non-decreasing ids");
      return BSM_E_INVALID;
    }
  }
  return BSM_OK;
}

// Key intervals in the index coordinate.  For key k of sample run S the legal
// query set is L = ((C u G) n Z) with C = tokens of S with 0 <= pos_q - pos_k
// < W, G = tokens of S with k's seg id (when it is >= 0), Z = tokens of S with
// k's noise id (all of S when it is < 0).  L is one run of indices exactly when
// |L| = max index - min index + 1; the planner computes |L| and its extreme
// indices from position-sorted token lists, and gives no range whenever it
// cannot (the kernels then test the four tracks, which is always exact).
struct RangeIndex {
  // tokens of one sample run sorted by (pos, index); sparse tables of the
  // indices' min and max over that order when positions do not rise with the
  // index (else the order is the index order and they are the ends)
  int64_t s0 = 0;
  bool rising = true;
  std::vector<int32_t> pos;  // ascending
  std::vector<int32_t> idx;
  std::vector<std::vector<int32_t>> mn, mx;

  void build(const Plan& p, int64_t a, int64_t b) {
    s0 = a;
    const int64_t n = b - a;
    rising = true;
    for (int64_t i = a + 1; i < b; ++i)
      if (p.pos[i] <= p.pos[i - 1]) rising = false;
    std::vector<std::pair<int32_t, int32_t>> v((size_t)n);
    for (int64_t i = 0; i < n; ++i) v[(size_t)i] = {p.pos[a + i], (int32_t)(a + i)};
    if (!rising) std::sort(v.begin(), v.end());
    pos.resize((size_t)n);
    idx.resize((size_t)n);
    for (int64_t i = 0; i < n; ++i) {
      pos[(size_t)i] = v[(size_t)i].first;
      idx[(size_t)i] = v[(size_t)i].second;
    }
    if (rising) return;
    mn.assign(1, idx);
    mx.assign(1, idx);
    for (int64_t w = 1; 2 * w <= n; w *= 2) {
      const std::vector<int32_t>&pm = mn.back(), &px = mx.back();
      std::vector<int32_t> nm((size_t)(n - 2 * w + 1)), nx((size_t)(n - 2 * w + 1));
      for (int64_t i = 0; i + 2 * w <= n; ++i) {
        nm[(size_t)i] = std::min(pm[(size_t)i], pm[(size_t)(i + w)]);
        nx[(size_t)i] = std::max(px[(size_t)i], px[(size_t)(i + w)]);
      }
      mn.push_back(std::move(nm));
      mx.push_back(std::move(nx));
    }
  }
  // min and max index over sorted positions [i0, i1), i1 > i0
  void extremes(int64_t i0, int64_t i1, int64_t& lo, int64_t& hi) const {
    if (rising) {
      lo = idx[(size_t)i0];
      hi = idx[(size_t)(i1 - 1)];
      return;
    }
    int l = 0;
    while ((int64_t(2) << l) <= i1 - i0) ++l;
    const int64_t j = i1 - (int64_t(1) << l);
    lo = std::min(mn[l][(size_t)i0], mn[l][(size_t)j]);
    hi = std::max(mx[l][(size_t)i0], mx[l][(size_t)j]);
  }
  // sorted-order range of positions [a, b)
  void span(int64_t a, int64_t b, int64_t& i0, int64_t& i1) const {
    i0 = std::lower_bound(pos.begin(), pos.end(), a, [](int32_t x, int64_t y) { return (int64_t)x < y; }) -
         pos.begin();
    i1 = std::lower_bound(pos.begin(), pos.end(), b, [](int32_t x, int64_t y) { return (int64_t)x < y; }) -
         pos.begin();
  }
};

// The tokens of one id (seg or noise) within one sample run.
struct IdSet {
  int64_t lo = INT64_MAX, hi = INT64_MIN, count = 0;
  std::vector<int32_t> pos;  // ascending (seg sets: for |C n G|)
  std::vector<int32_t> tok;  // token indices (noise sets: for the explicit scan)
  int32_t seg = INT32_MIN;   // noise sets: the seg id all tokens share, else INT32_MIN
  bool mixed = false;
};

uint64_t id_key(int64_t run, int32_t id) { return ((uint64_t)run << 32) | (uint32_t)id; }

constexpr int64_t kNoiseScan = 4096;  // explicit scan of a noise set up to this size

void key_interval(const Plan& p, int64_t k, const RangeIndex& ri, const IdSet* g, const IdSet* z,
                  int32_t& lo, int32_t& hi) {
  lo = 0;
  hi = -1;
  const int64_t pk = p.pos[k];
  const int64_t lim = pk + (int64_t)p.window;  // causal: pk <= pos_q < pk + W
  if (z && !(z->seg == p.seg[k] && p.seg[k] >= 0 && !z->mixed)) {
    // the noise set is not inside the key's seg: scan it (small sets only)
    if (z->count > kNoiseScan) return;
    int64_t c = 0, mn = INT64_MAX, mx = INT64_MIN;
    for (int32_t q : z->tok) {
      const int64_t pq = p.pos[q];
      if ((pq >= pk && pq < lim) || (p.seg[k] >= 0 && p.seg[q] == p.seg[k])) {
        ++c;
        mn = std::min<int64_t>(mn, q);
        mx = std::max<int64_t>(mx, q);
      }
    }
    if (c > 0 && c == mx - mn + 1) {
      lo = (int32_t)mn;
      hi = (int32_t)(mx + 1);
    }
    return;
  }
  int64_t count, mn, mx;
  if (z) {  // every token of the noise set is in the key's seg: L is the noise set
    count = z->count;
    mn = z->lo;
    mx = z->hi;
  } else {
    int64_t i0, i1;
    ri.span(pk, lim, i0, i1);
    count = i1 - i0;  // >= 1: the key itself
    ri.extremes(i0, i1, mn, mx);
    if (g) {
      const int64_t a = std::lower_bound(g->pos.begin(), g->pos.end(), pk,
                                         [](int32_t x, int64_t y) { return (int64_t)x < y; }) - g->pos.begin();
      const int64_t b = std::lower_bound(g->pos.begin(), g->pos.end(), lim,
                                         [](int32_t x, int64_t y) { return (int64_t)x < y; }) - g->pos.begin();
      count += g->count - (b - a);
      mn = std::min(mn, g->lo);
      mx = std::max(mx, g->hi);
    }
  }
  if (count == mx - mn + 1) {
    lo = (int32_t)mn;
    hi = (int32_t)(mx + 1);
  }
}

template <class F>
void parallel_for(int64_t count, int threads, F&& fn) {
  if (threads <= 1 || count < 2) {
    for (int64_t i = 0; i < count; ++i) fn(i);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> pool;
  const int nt = (int)std::min<int64_t>(threads, count);
  for (int t = 0; t < nt; ++t)
    pool.emplace_back([&] {
      for (;;) {
        const int64_t i = next.fetch_add(1);
        if (i >= count) break;
        fn(i);
      }
    });
  for (auto& th : pool) th.join();
}

}  // namespace

int build_plan(const bsm_plan_desc& d, Plan& p) {
  const auto t0 = std::chrono::steady_clock::now();
  int rc = validate(d);
  if (rc) return rc;
  p.n = d.n;
  p.ranks = d.ranks;
  p.block = d.block;
  p.order = d.order;
  p.window = d.window;
  p.shard = d.n / d.ranks;
  p.sample.assign(d.sample, d.sample + d.n);
  p.seg.assign(d.seg, d.seg + d.n);
  p.noise.assign(d.noise, d.noise + d.n);
  p.pos.assign(d.pos, d.pos + d.n);

  // tiles in the original order
  if (d.order == BSM_ORDER_CONTIGUOUS) {
    p.tps = (int32_t)((p.shard + d.block - 1) / d.block);
    for (int32_t r = 0; r < d.ranks; ++r)
      for (int32_t t = 0; t < p.tps; ++t) {
        const int64_t a = r * p.shard + (int64_t)t * d.block;
        p.tstart.push_back(a);
        p.tend.push_back(std::min(a + d.block, (r + 1) * p.shard));
      }
  } else {
    p.tps = (int32_t)(p.shard / d.block);
    for (int64_t a = 0; a < d.n; a += d.block) {
      p.tstart.push_back(a);
      p.tend.push_back(a + d.block);
    }
  }
  p.ntiles = (int32_t)p.tstart.size();
  const int32_t nt = p.ntiles;

  std::vector<Summary> sum(nt);
  for (int32_t t = 0; t < nt; ++t) sum[t] = summarize(p, p.tstart[t], p.tend[t]);

  // candidate key tile range [lo, hi) per query tile: sample ranges intersect
  std::vector<int32_t> smaxs(nt), smins(nt);
  for (int32_t t = 0; t < nt; ++t) {
    smins[t] = sum[t].smin;
    smaxs[t] = sum[t].smax;
  }
  int threads = d.threads;
  if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());

  std::vector<std::vector<int32_t>> rk(nt);
  std::vector<std::vector<int64_t>> rc_(nt);
  std::vector<std::vector<uint8_t>> rcl(nt);
  std::vector<int64_t> cand(nt, 0);
  parallel_for(nt, threads, [&](int64_t tq) {
    const Summary& qs = sum[tq];
    const int32_t lo = (int32_t)(std::lower_bound(smaxs.begin(), smaxs.end(), qs.smin) - smaxs.begin());
    const int32_t hi = (int32_t)(std::upper_bound(smins.begin(), smins.end(), qs.smax) - smins.begin());
    const int64_t qlen = p.tile_len((int32_t)tq);
    for (int32_t tk = lo; tk < hi; ++tk) {
      ++cand[tq];
      const int proof = prove(qs, sum[tk], p.window);
      if (proof < 0) continue;
      const int64_t full = qlen * p.tile_len(tk);
      const int64_t c = proof > 0 ? full
                                  : count_pairs(p, p.tstart[tq], p.tend[tq], p.tstart[tk], p.tend[tk]);
      if (c == 0) continue;
      rk[tq].push_back(tk);
      rc_[tq].push_back(c);
      rcl[tq].push_back(c == full ? BSM_TILE_FULL : BSM_TILE_PARTIAL);
    }
  });

  p.pptr.assign(nt + 1, 0);
  p.cost.assign(nt, 0);
  for (int32_t t = 0; t < nt; ++t) {
    p.pptr[t + 1] = p.pptr[t] + (int64_t)rk[t].size();
    p.candidates += cand[t];
  }
  p.pkey.resize(p.pptr[nt]);
  p.pcount.resize(p.pptr[nt]);
  p.pclass.resize(p.pptr[nt]);
  for (int32_t t = 0; t < nt; ++t) {
    std::copy(rk[t].begin(), rk[t].end(), p.pkey.begin() + p.pptr[t]);
    std::copy(rc_[t].begin(), rc_[t].end(), p.pcount.begin() + p.pptr[t]);
    std::copy(rcl[t].begin(), rcl[t].end(), p.pclass.begin() + p.pptr[t]);
    for (int64_t c : rc_[t]) p.cost[t] += c;
    for (uint8_t c : rcl[t]) (c == BSM_TILE_FULL ? p.nfull : p.npartial)++;
    p.total_pairs += p.cost[t];
  }

  // token order
  p.tiles_new.resize(nt);
  if (d.order == BSM_ORDER_CONTIGUOUS) {
    std::iota(p.tiles_new.begin(), p.tiles_new.end(), 0);
  } else if (d.order == BSM_ORDER_PTRR) {
    std::vector<int32_t> order(nt);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      return p.cost[a] != p.cost[b] ? p.cost[a] > p.cost[b] : a < b;
    });
    std::vector<int32_t> own(nt);
    for (int32_t i = 0; i < nt; ++i) {
      const int32_t round = i / d.ranks, slot = i % d.ranks;
      own[order[i]] = (round % 2 == 0) ? slot : d.ranks - 1 - slot;
    }
    int32_t k = 0;
    for (int32_t r = 0; r < d.ranks; ++r)
      for (int32_t t = 0; t < nt; ++t)
        if (own[t] == r) p.tiles_new[k++] = t;
  } else {
    std::vector<uint8_t> seen(nt, 0);
    for (int32_t i = 0; i < nt; ++i) {
      const int32_t t = d.explicit_block_perm[i];
      if (t < 0 || t >= nt || seen[t]) {
        set_error("explicit_block_perm is not a permutation of the blocks");
        return BSM_E_INVALID;
      }
      seen[t] = 1;
      p.tiles_new[i] = t;
    }
  }
  p.owner.resize(nt);
  p.local.resize(nt);
  for (int32_t i = 0; i < nt; ++i) {
    p.owner[p.tiles_new[i]] = i / p.tps;
    p.local[p.tiles_new[i]] = i % p.tps;
  }
  p.perm.clear();
  p.perm.reserve(d.n);
  for (int32_t i = 0; i < nt; ++i)
    for (int64_t x = p.tstart[p.tiles_new[i]]; x < p.tend[p.tiles_new[i]]; ++x) p.perm.push_back((int32_t)x);

  // key intervals (MARBLE section 03, "Block classification": a partial tile
  // can test one range per key instead of the full predicate)
  {
    p.pos_rising = true;
    for (int64_t i = 1; i < d.n; ++i)
      if (p.pos[i] <= p.pos[i - 1]) p.pos_rising = false;
    std::vector<std::pair<int64_t, int64_t>> runs;  // sample runs
    std::vector<int32_t> run_of(d.n);
    for (int64_t i = 0; i < d.n;) {
      int64_t j = i + 1;
      while (j < d.n && p.sample[j] == p.sample[i]) ++j;
      for (int64_t x = i; x < j; ++x) run_of[x] = (int32_t)runs.size();
      runs.push_back({i, j});
      i = j;
    }
    std::vector<RangeIndex> ri(runs.size());
    parallel_for((int64_t)runs.size(), threads, [&](int64_t r) { ri[r].build(p, runs[r].first, runs[r].second); });
    std::unordered_map<uint64_t, IdSet> segs, noises;
    for (int64_t i = 0; i < d.n; ++i) {
      if (p.seg[i] >= 0) {
        IdSet& g = segs[id_key(run_of[i], p.seg[i])];
        g.lo = std::min<int64_t>(g.lo, i);
        g.hi = std::max<int64_t>(g.hi, i);
        ++g.count;
        g.pos.push_back(p.pos[i]);
      }
      if (p.noise[i] >= 0) {
        IdSet& z = noises[id_key(run_of[i], p.noise[i])];
        z.lo = std::min<int64_t>(z.lo, i);
        z.hi = std::max<int64_t>(z.hi, i);
        if (z.count == 0) z.seg = p.seg[i];
        else if (z.seg != p.seg[i]) z.mixed = true;
        ++z.count;
        if (z.count <= kNoiseScan) z.tok.push_back((int32_t)i);
      }
    }
    for (auto& e : segs)
      if (!std::is_sorted(e.second.pos.begin(), e.second.pos.end()))
        std::sort(e.second.pos.begin(), e.second.pos.end());
    p.klo.assign(d.n, 0);
    p.khi.assign(d.n, -1);
    const int64_t chunk = 4096, nchunks = (d.n + chunk - 1) / chunk;
    parallel_for(nchunks, threads, [&](int64_t c) {
      const int64_t b = std::min(d.n, (c + 1) * chunk);
      for (int64_t k = c * chunk; k < b; ++k) {
        const int32_t run = run_of[k];
        const IdSet* g = p.seg[k] >= 0 ? &segs.at(id_key(run, p.seg[k])) : nullptr;
        const IdSet* z = p.noise[k] >= 0 ? &noises.at(id_key(run, p.noise[k])) : nullptr;
        key_interval(p, k, ri[run], g, z, p.klo[k], p.khi[k]);
      }
    });
    p.tile_kint.assign(nt, 1);
    p.interval_keys = 0;
    for (int32_t t = 0; t < nt; ++t)
      for (int64_t x = p.tstart[t]; x < p.tend[t]; ++x) {
        const bool ok = p.khi[x] >= p.klo[x];
        p.interval_keys += ok;
        if (!ok) p.tile_kint[t] = 0;
      }
  }

  // busiest rank: most legal pairs over all keys, ties -> lowest rank
  int64_t best = -1;
  for (int32_t r = 0; r < d.ranks; ++r) {
    int64_t tot = 0;
    for (int32_t a = 0; a < p.tps; ++a) tot += p.cost[p.tiles_new[r * p.tps + a]];
    if (tot > best) {
      best = tot;
      p.busiest = r;
    }
  }
  p.seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  return BSM_OK;
}

int vision_group_order(int64_t n, const int32_t* sample, const int32_t* seg, int32_t* out) {
  if (n < 1 || n > (int64_t(1) << 30)) { set_error("n must be in [1, 2^30]"); return BSM_E_INVALID; }
  if (!sample || !seg || !out) { set_error("null pointer"); return BSM_E_INVALID; }
  for (int64_t i = 0; i < n; ++i) {
    if (sample[i] < 0 || seg[i] < -1) { set_error("need sample >= 0 and seg >= -1"); return BSM_E_INVALID; }
    if (i > 0 && sample[i] < sample[i - 1]) {
      set_error("samples must be contiguous runs with non-decreasing ids");
      return BSM_E_INVALID;
    }
  }
  int64_t w = 0;
  std::vector<std::pair<int64_t, int64_t>> spans;  // runs of one seg id >= 0 in the sample
  std::unordered_map<int32_t, int32_t> nruns;      // seg id -> runs in the sample
  for (int64_t a = 0; a < n;) {
    int64_t b = a + 1;
    while (b < n && sample[b] == sample[a]) ++b;
    spans.clear();
    nruns.clear();
    for (int64_t i = a; i < b;) {
      int64_t j = i + 1;
      while (j < b && seg[j] == seg[i]) ++j;
      if (seg[i] >= 0) {
        spans.push_back({i, j});
        ++nruns[seg[i]];
      }
      i = j;
    }
    // a group: one seg id over two or more spans of the sample
    std::vector<uint8_t> in_group((size_t)(b - a), 0);
    std::vector<std::pair<int64_t, int64_t>> groups;
    for (const auto& sp : spans)
      if (nruns[seg[sp.first]] >= 2) {
        groups.push_back(sp);
        for (int64_t i = sp.first; i < sp.second; ++i) in_group[(size_t)(i - a)] = 1;
      }
    for (int64_t i = a; i < b; ++i)
      if (!in_group[(size_t)(i - a)]) out[w++] = (int32_t)i;
    for (auto it = groups.rbegin(); it != groups.rend(); ++it)
      for (int64_t i = it->first; i < it->second; ++i) out[w++] = (int32_t)i;
    a = b;
  }
  return BSM_OK;
}

int64_t step_map(const Plan& p, int32_t r, int32_t s, uint8_t* map) {
  const int32_t j = ((r - s) % p.ranks + p.ranks) % p.ranks;
  if (map) std::fill(map, map + (int64_t)p.tps * p.tps, (uint8_t)BSM_TILE_EMPTY);
  int64_t total = 0;
  for (int32_t a = 0; a < p.tps; ++a) {
    const int32_t tq = p.tiles_new[r * p.tps + a];
    for (int64_t e = p.pptr[tq]; e < p.pptr[tq + 1]; ++e) {
      const int32_t tk = p.pkey[e];
      if (p.owner[tk] != j) continue;
      if (map) map[(int64_t)a * p.tps + p.local[tk]] = p.pclass[e];
      total += p.pcount[e];
    }
  }
  return total;
}

int64_t fetch_set(const Plan& p, int32_t r, uint8_t* needed) {
  std::fill(needed, needed + (int64_t)p.ranks * p.tps, (uint8_t)0);
  int64_t count = 0;
  for (int32_t a = 0; a < p.tps; ++a) {
    const int32_t tq = p.tiles_new[r * p.tps + a];
    for (int64_t e = p.pptr[tq]; e < p.pptr[tq + 1]; ++e) {
      const int32_t tk = p.pkey[e];
      const int32_t j = p.owner[tk];
      if (j == r) continue;
      uint8_t& x = needed[(int64_t)j * p.tps + p.local[tk]];
      count += x == 0;
      x = 1;
    }
  }
  return count;
}

// Chunked ring attention (MARBLE section 03, "Chunked ring attention"): the
// sequence is cut into R*k contiguous chunks of whole tiles, k a power of two
// in [min_chunks, max_chunks] dividing the tiles per shard; chunks
// are dealt to ranks by the PTRR rule (sort, rounds of R, every other round
// reversed) once in the order of work and once in sequence order, optionally
// improved by greedy pairwise swaps of chunks between ranks; each rank keeps
// its tiles in sequence order.  The cost of a layout is
//   C = sum_s max_r W[r][(r - s) mod R] + tau * R * k,
// with W[r][j] the legal pairs between rank r's queries and rank j's keys
// (from the exact tile-pair counts) and tau the fixed cost of one range in one
// step, in pairs.  The cheapest candidate wins (ties: fewer chunks, then work
// order).
namespace {

struct ChunkEval {
  const Plan& p;
  int32_t R, k, nchunks, ctiles;
  std::vector<int32_t> tile_chunk;  // original tile -> chunk
  std::vector<int64_t> cpair;       // chunk x chunk legal pairs
  ChunkEval(const Plan& p_, int32_t k_) : p(p_), R(p_.ranks), k(k_) {
    nchunks = R * k;
    ctiles = p.ntiles / nchunks;
    tile_chunk.resize(p.ntiles);
    for (int32_t t = 0; t < p.ntiles; ++t) tile_chunk[t] = t / ctiles;
    cpair.assign((size_t)nchunks * nchunks, 0);
    for (int32_t tq = 0; tq < p.ntiles; ++tq)
      for (int64_t e = p.pptr[tq]; e < p.pptr[tq + 1]; ++e)
        cpair[(size_t)tile_chunk[tq] * nchunks + tile_chunk[p.pkey[e]]] += p.pcount[e];
  }
  // sum over steps of the slowest rank, for chunk -> rank assignment `own`
  double step_max_sum(const std::vector<int32_t>& own) const {
    std::vector<int64_t> w((size_t)R * R, 0);
    for (int32_t a = 0; a < nchunks; ++a)
      for (int32_t b = 0; b < nchunks; ++b) w[(size_t)own[a] * R + own[b]] += cpair[(size_t)a * nchunks + b];
    double tot = 0;
    for (int32_t s = 0; s < R; ++s) {
      int64_t mx = 0;
      for (int32_t r = 0; r < R; ++r) mx = std::max(mx, w[(size_t)r * R + ((r - s) % R + R) % R]);
      tot += (double)mx;
    }
    return tot;
  }
};

// PTRR dealing of chunks given in `order` (rounds of R, odd rounds reversed).
std::vector<int32_t> deal(const std::vector<int32_t>& order, int32_t R) {
  std::vector<int32_t> own(order.size());
  for (size_t i = 0; i < order.size(); ++i) {
    const int32_t round = (int32_t)(i / R), slot = (int32_t)(i % R);
    own[order[i]] = (round % 2 == 0) ? slot : R - 1 - slot;
  }
  return own;
}

}  // namespace

int chunk_order(const Plan& p, int32_t min_chunks, int32_t max_chunks, double tau, int32_t swaps,
                int32_t* block_perm, ChunkResult& out) {
  const int32_t R = p.ranks;
  if (p.n % ((int64_t)p.block * R)) {  // an explicit block order needs whole blocks per rank
    set_error("chunked layouts need n % (block * ranks) == 0");
    return BSM_E_INVALID;
  }
  if (min_chunks < 1 || max_chunks < min_chunks || swaps < 0 || !(tau >= 0)) {
    set_error("need 1 <= min_chunks <= max_chunks, swaps >= 0, tau >= 0");
    return BSM_E_INVALID;
  }
  const int32_t tps = p.ntiles / R;
  bool found = false;
  std::vector<int32_t> best_own;
  int32_t best_k = 0;
  for (int32_t k = 1; k <= max_chunks && k <= tps; k *= 2) {
    if (k < min_chunks || tps % k) continue;
    ChunkEval ev(p, k);
    std::vector<int64_t> work(ev.nchunks, 0);
    for (int32_t a = 0; a < ev.nchunks; ++a)
      for (int32_t b = 0; b < ev.nchunks; ++b) work[a] += ev.cpair[(size_t)a * ev.nchunks + b];
    for (int32_t strategy = 0; strategy < 2; ++strategy) {
      std::vector<int32_t> order(ev.nchunks);
      std::iota(order.begin(), order.end(), 0);
      if (strategy == 0)
        std::stable_sort(order.begin(), order.end(),
                         [&](int32_t a, int32_t b) { return work[a] != work[b] ? work[a] > work[b] : a < b; });
      std::vector<int32_t> own = deal(order, R);
      double cur = ev.step_max_sum(own);
      // greedy pairwise swaps of chunks on different ranks, first improvement
      // (quartic in the chunk count: only for up to 64 chunks)
      for (int32_t pass = 0; pass < (ev.nchunks <= 64 ? swaps : 0); ++pass) {
        bool improved = false;
        for (int32_t a = 0; a < ev.nchunks && !improved; ++a)
          for (int32_t b = a + 1; b < ev.nchunks && !improved; ++b) {
            if (own[a] == own[b]) continue;
            std::swap(own[a], own[b]);
            const double c = ev.step_max_sum(own);
            if (c < cur) {
              cur = c;
              improved = true;
            } else {
              std::swap(own[a], own[b]);
            }
          }
        if (!improved) break;
      }
      const double range_term = tau * R * k;
      const double cost = cur + range_term;
      if (!found || cost < out.cost) {
        found = true;
        out.cost = cost;
        out.step_max_sum = cur;
        out.range_term = range_term;
        out.chunks_per_rank = k;
        out.strategy = strategy;
        best_own = own;
        best_k = k;
      }
    }
  }
  if (!found) {
    set_error("no chunk count divides the tiles per shard");
    return BSM_E_INVALID;
  }
  // explicit block order: ranks in order, each rank's tiles ascending
  const int32_t ctiles = p.ntiles / (R * best_k);
  int32_t pos = 0;
  for (int32_t r = 0; r < R; ++r)
    for (int32_t t = 0; t < p.ntiles; ++t)
      if (best_own[t / ctiles] == r) block_perm[pos++] = t;
  return BSM_OK;
}

}  // namespace bsm
