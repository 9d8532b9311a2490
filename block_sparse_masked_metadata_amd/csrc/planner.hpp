// Host planner internals shared by planner.cpp and capi.cpp (C++17, no HIP).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "bsm.h"

namespace bsm {

// Per-thread error text behind bsm_last_error().
void set_error(const std::string& msg);

struct Plan {
  int64_t n = 0;
  int32_t ranks = 1, block = 128, order = 0, window = BSM_WINDOW_INF;
  int64_t shard = 0;            // tokens per shard
  int32_t tps = 0;              // tiles per shard
  int32_t ntiles = 0;           // ranks * tps
  // tiles in the ORIGINAL order: [tstart, tend)
  std::vector<int64_t> tstart, tend;
  std::vector<int32_t> tiles_new;  // new tile position -> original tile
  std::vector<int32_t> owner;      // original tile -> shard
  std::vector<int32_t> local;      // original tile -> index in its shard
  std::vector<int64_t> cost;       // legal pairs of the tile's queries
  // non-empty tile pairs, CSR over original query tiles, ascending key tile
  std::vector<int64_t> pptr;
  std::vector<int32_t> pkey;
  std::vector<int64_t> pcount;
  std::vector<uint8_t> pclass;
  std::vector<int32_t> perm;       // new token -> original token
  // tracks, original order
  std::vector<int32_t> sample, seg, noise, pos;
  // Key intervals, original order: the queries key k is legal for are exactly
  // the tokens with index in [klo[k], khi[k]) (index in the caller's order),
  // or the key has no such range (khi < klo).
  std::vector<int32_t> klo, khi;
  bool pos_rising = true;          // positions rise strictly with the index
  std::vector<uint8_t> tile_kint;  // original tile: every key has an interval
  int64_t interval_keys = 0;
  int32_t busiest = 0;
  int64_t total_pairs = 0, candidates = 0, nfull = 0, npartial = 0;
  double seconds = 0;

  int64_t tile_len(int32_t t) const { return tend[t] - tstart[t]; }
};

// Build; returns BSM_OK or an error code (error text set).
int build_plan(const bsm_plan_desc& desc, Plan& out);

// Vision-group token order of a packed sequence (see bsm.h); out[i] = the
// index of the token placed at position i.
int vision_group_order(int64_t n, const int32_t* sample, const int32_t* seg, int32_t* out);

// Legal pairs of rank r at step s and optional tile map.
int64_t step_map(const Plan& p, int32_t r, int32_t s, uint8_t* map);

// Sparse fetch: needed[j * tps + b] = 1 when some query tile of rank r has a
// non-empty pair with key tile b of shard j != r; returns the number of such
// remote tiles.
int64_t fetch_set(const Plan& p, int32_t r, uint8_t* needed);

// Chunked ring layout (see planner.cpp): the explicit block order of the
// cheapest candidate and its cost terms.
struct ChunkResult {
  int32_t chunks_per_rank = 0, strategy = 0;
  double cost = 0, step_max_sum = 0, range_term = 0;
};
int chunk_order(const Plan& p, int32_t min_chunks, int32_t max_chunks, double tau, int32_t swaps,
                int32_t* block_perm, ChunkResult& out);

// Dense calls of rank r at step s (see calls.cpp): query rows [q0, q0 + qn)
// of rank r's shard against key rows [k0, k0 + kn) of shard (r - s) mod R,
// every pair of whose positions satisfies the relation `kind` computed.
enum : int32_t { kCallFull = 0, kCallCausal = 1, kCallReverse = 2, kCallPastWindow = 3 };
struct Call {
  int32_t q0, qn, k0, kn, kind;
};
int dense_calls(const Plan& p, int32_t r, int32_t s, std::vector<Call>& out);
// 0: no pair of the position bounds satisfies relation `kind`, 2: every
// pair does, 1: some may.
int relation_bounds(int32_t kind, int64_t qmin, int64_t qmax, int64_t kmin, int64_t kmax, int64_t w);

}  // namespace bsm

struct bsm_plan {
  bsm::Plan p;
};
