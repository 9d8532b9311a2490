// Dense calls of one ring step (MARBLE section 03, "Chunked ring attention":
// every ring step runs as a few dense calls instead of a masked block-sparse
// one; each legal pair is computed by exactly one call).
//
// A call pairs a run of the rank's query rows with a run of the step's key
// rows (both in plan order, local to their shards) and one relation between
// their positions:
//   full         every pair
//   causal       0 <= pos_q - pos_k < W   (W = the layer's window)
//   reverse      pos_k > pos_q
//   past window  pos_q - pos_k >= W       (only for a finite window)
// The calls come from four families of token sets; every legal pair falls in
// exactly one family and one relation, because
//   legal = same sample and (causal or same seg >= 0) and (noise_k < 0 or noise_q == noise_k):
//   A  queries of sample x,            clean keys of x             causal
//   B  queries of seg g (g >= 0),      clean keys of g             reverse, past window
//   C  queries of noise span z,        keys of z                   causal (full when every
//                                                                  token of z has one seg >= 0)
//   D  queries of z with seg g,        keys of z with seg g        reverse, past window
//                                                                  (not when C is full)
// A clean key (noise < 0) is legal for a query of its sample iff the pair is
// causal (A) or, failing that, shares a seg (B: the non-causal rest of a seg
// is the keys after the query plus those past the window).  A noise key is
// legal only for queries of its own span, by the same split (C, D).
// Samples, segs and noise spans are the page's mask tracks.

#include <algorithm>
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "planner.hpp"

namespace bsm {
namespace {

struct Key {
  int32_t a = 0, b = 0, c = 0;
  bool operator==(const Key& o) const { return a == o.a && b == o.b && c == o.c; }
  bool operator<(const Key& o) const {
    return a != o.a ? a < o.a : b != o.b ? b < o.b : c < o.c;
  }
};

struct RunRec {
  Key key;
  int32_t start, end;      // local rows [start, end)
  int32_t pmin, pmax;      // position bounds of its rows
};

// Maximal runs of consecutive local rows [0, S) of the shard starting at plan
// row `base` whose tokens are in the family (fam returns false otherwise) with
// one family key.
template <class F>
std::vector<RunRec> family_runs(const Plan& p, int64_t base, int64_t S, F fam) {
  std::vector<RunRec> out;
  for (int64_t i = 0; i < S; ++i) {
    const int32_t t = p.perm[base + i];
    Key k;
    if (!fam(t, k)) continue;
    const int32_t pos = p.pos[t];
    if (!out.empty() && out.back().end == i && out.back().key == k) {
      RunRec& r = out.back();
      r.end = (int32_t)i + 1;
      r.pmin = std::min(r.pmin, pos);
      r.pmax = std::max(r.pmax, pos);
    } else {
      out.push_back({k, (int32_t)i, (int32_t)i + 1, pos, pos});
    }
  }
  std::stable_sort(out.begin(), out.end(), [](const RunRec& x, const RunRec& y) { return x.key < y.key; });
  return out;
}

}  // namespace

int relation_bounds(int32_t kind, int64_t qmin, int64_t qmax, int64_t kmin, int64_t kmax, int64_t w) {
  bool all = false, none = false;
  switch (kind) {
    case kCallCausal:
      all = qmin - kmax >= 0 && qmax - kmin < w;
      none = qmax - kmin < 0 || qmin - kmax >= w;
      break;
    case kCallReverse:
      all = kmin > qmax;
      none = kmax <= qmin;
      break;
    case kCallPastWindow:
      all = qmin - kmax >= w;
      none = qmax - kmin < w;
      break;
    default:
      all = true;
  }
  return none ? 0 : all ? 2 : 1;
}

int dense_calls(const Plan& p, int32_t r, int32_t s, std::vector<Call>& out) {
  out.clear();
  // the relations of a call compare positions over runs of rows, which
  // needs positions that rise with the token index
  if (!p.pos_rising) {
    set_error("dense calls need positions that rise with the token index");
    return BSM_E_UNSUPPORTED;
  }
  const int32_t R = p.ranks;
  const int32_t j = ((r - s) % R + R) % R;
  const int64_t S = p.shard, qbase = (int64_t)r * S, kbase = (int64_t)j * S;
  const bool finite = p.window < BSM_WINDOW_INF;

  // (sample, noise) -> the one seg >= 0 every token of that noise span has, or -2
  std::unordered_map<uint64_t, int32_t> uniform;
  auto nkey = [](int32_t smp, int32_t z) { return ((uint64_t)(uint32_t)smp << 32) | (uint32_t)z; };
  for (int64_t t = 0; t < p.n; ++t) {
    if (p.noise[t] < 0) continue;
    auto it = uniform.find(nkey(p.sample[t], p.noise[t]));
    if (it == uniform.end())
      uniform.emplace(nkey(p.sample[t], p.noise[t]), p.seg[t] >= 0 ? p.seg[t] : -2);
    else if (it->second != p.seg[t])
      it->second = -2;
  }
  auto unif = [&](int32_t t) { return uniform.at(nkey(p.sample[t], p.noise[t])); };

  // one family: query runs x key runs with equal keys, each call pruned by its
  // run bounds (a relation no pair satisfies gives no call; one every pair
  // satisfies gives a full call)
  auto emit = [&](const std::vector<RunRec>& qr, const std::vector<RunRec>& kr, const int32_t* kinds, int nk) {
    size_t a = 0, b = 0;
    while (a < qr.size() && b < kr.size()) {
      if (qr[a].key < kr[b].key) { ++a; continue; }
      if (kr[b].key < qr[a].key) { ++b; continue; }
      size_t a1 = a, b1 = b;
      while (a1 < qr.size() && qr[a1].key == qr[a].key) ++a1;
      while (b1 < kr.size() && kr[b1].key == kr[b].key) ++b1;
      for (size_t x = a; x < a1; ++x)
        for (size_t y = b; y < b1; ++y)
          for (int i = 0; i < nk; ++i) {
            const int c = relation_bounds(kinds[i], qr[x].pmin, qr[x].pmax, kr[y].pmin, kr[y].pmax, p.window);
            if (c == 0) continue;
            out.push_back({qr[x].start, qr[x].end - qr[x].start, kr[y].start, kr[y].end - kr[y].start,
                           c == 2 ? (int32_t)kCallFull : kinds[i]});
          }
      a = a1;
      b = b1;
    }
  };
  const int32_t kCausal[1] = {kCallCausal};
  const int32_t kRest[2] = {kCallReverse, kCallPastWindow};
  const int nrest = finite ? 2 : 1;

  // A: sample x clean keys, causal
  {
    auto fq = [&](int32_t t, Key& k) { k = {p.sample[t], 0, 0}; return true; };
    auto fk = [&](int32_t t, Key& k) { k = {p.sample[t], 0, 0}; return p.noise[t] < 0; };
    emit(family_runs(p, qbase, S, fq), family_runs(p, kbase, S, fk), kCausal, 1);
  }
  // B: seg g x clean keys of g, the non-causal rest
  {
    auto fq = [&](int32_t t, Key& k) { k = {p.sample[t], p.seg[t], 0}; return p.seg[t] >= 0; };
    auto fk = [&](int32_t t, Key& k) { k = {p.sample[t], p.seg[t], 0}; return p.seg[t] >= 0 && p.noise[t] < 0; };
    emit(family_runs(p, qbase, S, fq), family_runs(p, kbase, S, fk), kRest, nrest);
  }
  // C: noise span z x keys of z (full for spans of one seg, else causal)
  {
    auto fq = [&](int32_t t, Key& k) {
      if (p.noise[t] < 0) return false;
      k = {p.sample[t], p.noise[t], unif(t) >= 0 ? 1 : 0};
      return true;
    };
    auto fk = fq;
    const auto qr = family_runs(p, qbase, S, fq), kr = family_runs(p, kbase, S, fk);
    // spans of one seg: every pair is legal
    std::vector<RunRec> qf, kf, qc, kc;
    for (auto& x : qr) (x.key.c ? qf : qc).push_back(x);
    for (auto& x : kr) (x.key.c ? kf : kc).push_back(x);
    const int32_t kFullKind[1] = {kCallFull};
    emit(qf, kf, kFullKind, 1);
    emit(qc, kc, kCausal, 1);
  }
  // D: (z, g) of spans with several segs, the non-causal rest
  {
    auto f = [&](int32_t t, Key& k) {
      k = {p.sample[t], p.noise[t], p.seg[t]};
      return p.noise[t] >= 0 && p.seg[t] >= 0 && unif(t) < 0;
    };
    emit(family_runs(p, qbase, S, f), family_runs(p, kbase, S, f), kRest, nrest);
  }
  return BSM_OK;
}

}  // namespace bsm
