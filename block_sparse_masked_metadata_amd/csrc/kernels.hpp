// Device-side data layout and kernel launchers (internal to libbsm.so).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace bsm {

constexpr int kHeadDim = 128;   // d
constexpr int kTile = 128;      // query and key tile tokens

// Work item of a list-driven kernel (int4 in device memory):
//   x = query tile index (forward / dQ), or the first key row of the key tile
//       (dK/dV column items: the tiles of a compact sparse-fetch buffer start
//       at any row, not only at multiples of 128)
//   y = flags (kFirst: the tile's first step with work, kLast: its last)
//   z = first entry of the tile's list, w = number of entries
//   kKeyInterval (backward column items): every key of the tile has a key
//   interval, so partial pairs test lo <= pos_q < hi
//   Backward column items also carry the key tile's valid rows (1..128) in
//   bits kKeyRowsShift.. of y: a tile of a compact sparse-fetch buffer can be
//   ragged in the middle of the buffer, so the row count cannot come from the
//   buffer's length.
enum : int32_t { kFirst = 1, kLast = 2, kKeyInterval = 4 };
constexpr int kKeyRowsShift = 8;
__host__ __device__ inline int32_t key_rows(int32_t y) { return (y >> kKeyRowsShift) & 0xff; }

// List entry (int2): x = first row of the partner tile in the partner buffer,
//                    y = valid rows of the partner tile | (partial << 16)
// A partner tile with fewer than 128 valid rows is always marked partial.
// kIntervalBit (with the partial bit, forward and dQ lists): every key of the
// partner tile has a key interval.
constexpr int32_t kPartialBit = 1 << 16;
constexpr int32_t kIntervalBit = 1 << 17;
constexpr int32_t kLenMask = 0xff;  // valid rows: at most 128
// Dense-call entries (forward lists of a dense-call device plan): the entry
// applies to query rows [lo, hi] of its tile, lo in bits 8-14 and hi in bits
// 24-30, and bits 19-20 hold the relation its pairs satisfy (kCallFull,
// kCallCausal, kCallReverse or kCallPastWindow of the planner).  With the
// partial bit the kernel tests row range and relation (one compare per pair),
// and masks keys past the valid rows.
constexpr int kRowLoShift = 8, kRowHiShift = 24, kKindShift = 19;
enum : int32_t { kRelFull = 0, kRelCausal = 1, kRelReverse = 2, kRelPastWindow = 3 };
// Column entries of a dense-call plan (dK/dV lists) mirror this: x = first
// query row, the rows [lo, hi] bits name the KEY rows of the key tile the
// entry applies to.

// Dense-call masks as one range per lane (branch-free: a branch on the
// relation splits the kernels' loops and costs registers).  Positions lie in
// [0, 2^31 - 1) and 1 <= window <= 2^31 - 1, so the signed arithmetic below
// does not overflow.  A lane tests a position x with the unsigned difference
// (uint32_t)x - (uint32_t)lo < span (modulo 2^32, well defined also for
// lo = INT32_MIN); the pad position INT32_MAX of keys past a ragged tile's
// valid rows lies outside every range, since no range reaches 2^31 - 1.
// Query lane (forward, dQ): the key positions legal for query row `row` of
// its tile at position pq under entry word y are [lo, lo + span).
__device__ inline void dense_range(int32_t y, int row, int32_t pq, int32_t window, int32_t& lo, uint32_t& span) {
  const int kind = (y >> kKindShift) & 3;
  const int rlo = (y >> kRowLoShift) & 127, rhi = ((y >> kRowHiShift) & 127) + 1;
  const int32_t below = pq - window + 1;
  lo = kind == kRelCausal ? below : kind == kRelReverse ? pq + 1 : INT32_MIN;
  const int32_t hi = kind == kRelCausal ? pq + 1 : kind == kRelPastWindow ? below : INT32_MAX;
  span = (uint32_t)(row - rlo) < (uint32_t)(rhi - rlo) ? (uint32_t)hi - (uint32_t)lo : 0u;
}
// Key lane (dK/dV): the query positions legal for key row `row` of its tile
// at position pk under column entry word y are [lo, lo + span).
__device__ inline void dense_key_range(int32_t y, int row, int32_t pk, int32_t window, int32_t& lo, uint32_t& span) {
  const int kind = (y >> kKindShift) & 3;
  const int rlo = (y >> kRowLoShift) & 127, rhi = ((y >> kRowHiShift) & 127) + 1;
  const int32_t ahead = window > INT32_MAX - pk ? INT32_MAX : pk + window;  // pk + W, saturated
  lo = kind == kRelCausal ? pk : kind == kRelPastWindow ? ahead : INT32_MIN;
  const int32_t hi = kind == kRelCausal ? ahead : kind == kRelReverse ? pk : INT32_MAX;
  span = (uint32_t)(row - rlo) < (uint32_t)(rhi - rlo) ? (uint32_t)hi - (uint32_t)lo : 0u;
}

// Key interval of a token (int2): the queries it is legal for are exactly
// those whose index in the caller's token order lies in [x, y); y < x when it
// has none (the planner's key_interval).  The device plan carries that index
// per plan row (`coord`), the coordinate the kernels test it against.

// The carried forward state O_acc is tile-blocked (each workgroup's state is
// one contiguous 64 KiB run that its lanes read and write fully coalesced):
// query tile t = row / 128 and head h own 128 x 128 floats at
// (t * Hq + h) * 16384; inside, wave w = (row % 128) / 32 owns 4096 floats,
// and the lane of query row 32w + l (l < 32) for channel d = 32 db + 8 i +
// 4 hi + c keeps it at float (64 (4 db + i) + l + 32 hi) * 4 + c.  A buffer
// holds ceil(S / 128) * 128 * Hq * 128 floats.
__host__ __device__ inline int64_t state_index(int64_t row, int32_t h, int32_t d, int32_t hq) {
  const int64_t t = row >> 7;
  const int r = (int)(row & 127), w = r >> 5, l = r & 31;
  const int db = d >> 5, i = (d >> 3) & 3, hi = (d >> 2) & 1, c = d & 3;
  return (t * hq + h) * (int64_t)(kTile * kHeadDim) + w * 32 * kHeadDim + (((db * 4 + i) * 64 + l + 32 * hi) << 2) + c;
}

// Per-token tracks in plan order (int4): sample, seg, noise, pos.
// bf16 tensors are passed as raw 16-bit patterns (uint16_t).

struct FwdArgs {
  const int4* items;
  const int2* first;        // items[i]'s first list entry (entries[items[i].z])
  const int2* entries;
  int32_t nitems;
  int32_t hq, hkv;
  int32_t heads_per_xcd;   // >0: XCD-aware block->(item, head) map
  const uint16_t* q;  // [S, Hq, d]
  const uint16_t* k;  // [*, Hkv, d]
  const uint16_t* v;
  const int4* qtracks;      // tracks of the query shard rows
  const int32_t* qcoord;    // key-interval coordinate of the query shard rows
  const int4* ktracks;      // tracks of the key buffer rows
  const int2* kint;         // key intervals of the key buffer rows
  int64_t rows;             // S: query shard rows (state stride / ragged bound)
  float* oacc;              // tile-blocked fp32 (state_index)
  float* m;                 // [Hq, S]
  float* l;                 // [Hq, S]
  uint16_t* o;        // [S, Hq, d]
  float* lse;               // [Hq, S]
  float scale_log2;         // scale * log2(e)
  int32_t window;
  int32_t keep_state;
  int32_t step_only;        // ignore the carried state and finalize every item
  int32_t dense;            // the lists hold dense-call entries
};

struct BwdArgs {
  const int4* items;
  const int2* entries;
  int32_t nitems;
  int32_t hq, hkv;
  int32_t heads_per_xcd;
  const uint16_t* q;    // [S, Hq, d]
  const uint16_t* k;    // [Sk, Hkv, d]
  const uint16_t* v;
  const uint16_t* dout; // [S, Hq, d]
  const float* lse;           // [Hq, S] natural log
  const float* delta;         // [Hq, S]
  const int4* qtracks;
  const int32_t* qcoord;      // key-interval coordinate of the query shard rows
  const int4* ktracks;
  const int2* kint;           // key intervals of the key buffer rows
  int32_t dense;              // the lists hold dense-call entries
  int64_t rows;               // S (query rows)
  int64_t krows;              // key rows of the k/v buffers
  float* dq;                  // [S, Hq, d]
  float* dk;                  // [Sk, Hkv, d]
  float* dv;
  float scale;                // softmax scale
  float scale_log2;
  int32_t window;
  // split dK/dV work (nullable): work units int4 {item, first sub-tile, end
  // sub-tile, workspace slot or -1}; nitems counts the units.  A unit with a
  // slot writes its scaled partial dK, dV of the tile to workspace slot
  // (slot * Hkv + kv head) as two [128 keys][128] fp32 blocks; a unit without
  // one adds into dk / dv.
  const int4* work;
  float* ws;
  // reduction after a split launch: int4 {first key row of the tile, first
  // slot, slots, valid rows of the key tile}
  const int4* reduce;
  int32_t nreduce;
};

// Sparse fetch, the way back: dk_all[src[c]] += dk_fetch[c] (and dV) for every
// row c of the compact buffer with src[c] >= 0, all key/value heads.
struct FetchAccArgs {
  const int32_t* src;    // [fetch_rows] shard row (plan order) or -1
  int64_t rows;          // fetch_rows
  int32_t hkv;
  const float* dk_fetch;
  const float* dv_fetch;
  float* dk;             // [R * S, Hkv, d]
  float* dv;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// Accuracy controls: merge one step's partial result into a running one.
hipError_t launch_merge_bf16(int64_t rows, int32_t hq, uint16_t* o_run, float* lse_run, const uint16_t* o_s,
                             const float* lse_s, hipStream_t stream);
hipError_t launch_merge_fp32(int64_t rows, int32_t hq, float* o_run, float* lse_run, const float* acc_s,
                             const float* m_s, const float* l_s, uint16_t* o_bf16, hipStream_t stream);
// O_acc (tile-blocked) -> fp32 [rows, Hq, d].
hipError_t launch_state_unpack(int64_t rows, int32_t hq, const float* o_acc, float* out, hipStream_t stream);
hipError_t launch_bwd_prep(int64_t rows, int32_t hq, const uint16_t* o,
                           const uint16_t* dout, float* delta, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fetch_accumulate(const FetchAccArgs& a, hipStream_t stream);
// dk/dv rows of every reduce entry's key tile += its workspace slots, in slot order.
hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t stream);

}  // namespace bsm
