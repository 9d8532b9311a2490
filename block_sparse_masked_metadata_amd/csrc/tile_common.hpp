// Device helpers shared by the forward and backward kernels (gfx950).
#pragma once

#include "kernels.hpp"

namespace bsm {
namespace dev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kNegInf = -__builtin_inff();
constexpr float kInf = __builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kSub = 64;  // rows per staged sub-tile (half of a listed 128-row tile)

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline f32x16 mfma(const bf16x8 a, const bf16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two LDS transpose reads (ds_read_b64_tr_b16) -> one 8-element MFMA operand.
// In each 16-lane group, lane l receives element l%4 of the 8 bytes addressed
// by lane 4e + l/4 of its group, for e = 0..3.
__device__ inline bf16x8 lds_tr8(const char* p0, const char* p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// The mask predicate of MARBLE section 01 over per-token tracks (x = sample,
// y = seg, z = noise, w = pos).  The query side must come through
// query_tracks(): a negative query seg becomes -2, which no key seg (>= -1)
// equals, so seg equality alone means "same span" (seg_q == seg_k >= 0).
// Positions lie in [-1, 2^31 - 1) (-1 only on pad rows), so pos_q - pos_k
// does not overflow, and as an unsigned number it is below the window
// exactly when 0 <= pos_q - pos_k < window.
__device__ inline int4 query_tracks(int4 q) {
  q.y = q.y < 0 ? -2 : q.y;
  return q;
}
__device__ inline bool legal(const int4 q, const int4 k, int32_t window) {
  const uint32_t d = (uint32_t)(q.w - k.w);
  return ((d < (uint32_t)window) | (q.y == k.y)) & ((k.z < 0) | (q.z == k.z)) & (q.x == k.x);
}

// Workgroup -> (list item, head).  Workgroups are dispatched round-robin over
// the 8 XCDs; with hpx > 0 XCD x gets heads [x*hpx, (x+1)*hpx) (so a head's
// tiles stay in one L2) and walks its items in list order, heads inner.
__device__ inline void map_block(int32_t b, int32_t nitems, int32_t heads, int32_t hpx,
                                 int32_t& item, int32_t& h) {
  if (hpx > 0) {
    const int32_t x = b & 7, i = b >> 3;
    item = i / hpx;
    h = x * hpx + i % hpx;
  } else {
    item = b / heads;
    h = b % heads;
  }
  if (item >= nitems) item = -1;
}

// ---- staged 64 x 128 bf16 tiles: rows of 256 B, 16-byte chunks XOR-swizzled ----
// Chunk c of row r sits in slot c ^ f(r), f(r) = 4(r & 3) + ((r >> 2) & 3).
// f is a bijection on any 16 consecutive rows, so MFMA operand reads of one
// chunk over 16 rows hit 16 distinct slots; and for the transpose reads (rows
// r0..r0+3, r0 % 4 == 0, chunks 4j..4j+3) the slots c ^ f(r) fall in four
// disjoint groups of four.  Both access patterns are bank-conflict free.
__device__ inline int tile_slot(int r, int c) {
  return r * 256 + ((c ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 4);
}

// Per-lane constants of the transpose reads of a staged tile: the A operand
// of an MFMA over 16 tile rows starting at row `r16`, output rows = the 32
// channels [32 db, 32 db + 32).  Row slots permute 16 keys as the MFMA
// accumulator layout of S^T requires (see the forward kernel's header).
struct TrLane {
  int row0, chunk, off8;
  __device__ inline explicit TrLane(int lane) {
    const int G = lane >> 4, jl = lane & 15;
    row0 = 4 * (G >> 1) + (jl >> 2);
    chunk = 2 * (G & 1) + ((jl & 3) >> 1);
    off8 = (jl & 1) * 8;
  }
  __device__ inline bf16x8 read(const char* tile, int r16, int db) const {
    const int r = r16 + row0;
    return lds_tr8(tile + tile_slot(r, 4 * db + chunk) + off8, tile + tile_slot(r + 8, 4 * db + chunk) + off8);
  }
};

// MFMA operand of row `row`, channels [16 kk + 8 hi, +8) of a staged tile.
__device__ inline bf16x8 row_operand(const char* tile, int row, int kk, int hi) {
  return as_bf16x8(*(const uint4*)(tile + tile_slot(row, 2 * kk + hi)));
}

// Two 64-row sub-tiles (A and B, e.g. K and V) staged through registers:
// thread t holds chunk t%16 of rows t/16 + 16i (i = 0..3), so every 16 lanes
// read one 256-byte row contiguously.  Rows past `len` are zero.
struct PairStage {
  uint4 a[4], b[4];
  // abytes/bbytes: uniform base addresses; byte offsets stay below 2^32.
  __device__ inline void fetch(const char* abytes, const char* bbytes, int64_t r0, int len,
                               uint32_t row_bytes, int tid) {
    const uint32_t off = (uint32_t)(r0 + (tid >> 4)) * row_bytes + (uint32_t)(tid & 15) * 16u;
    if (len == kSub) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = *(const uint4*)(abytes + (off + 16u * i * row_bytes));
        b[i] = *(const uint4*)(bbytes + (off + 16u * i * row_bytes));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 4) + 16 * i;
        a[i] = make_uint4(0, 0, 0, 0);
        b[i] = make_uint4(0, 0, 0, 0);
        if (row < len) {
          a[i] = *(const uint4*)(abytes + (off + 16u * i * row_bytes));
          b[i] = *(const uint4*)(bbytes + (off + 16u * i * row_bytes));
        }
      }
    }
  }
  __device__ inline void store(char* ta, char* tb, int tid) const {
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 4) + 16 * i;
      *(uint4*)(ta + tile_slot(row, c)) = a[i];
      *(uint4*)(tb + tile_slot(row, c)) = b[i];
    }
  }
};

// Sub-tile n of a list item: half n%2 of list entry n/2 (entry: first row of
// the partner tile, valid rows | partial bit << 16).
__device__ inline void sub_bounds(const int2 ent, int n, int64_t& r0, int& len, bool& partial) {
  const int half = n & 1;
  const int tlen = ent.y & kLenMask;
  r0 = (int64_t)ent.x + half * kSub;
  len = tlen - half * kSub;
  len = len < 0 ? 0 : (len > kSub ? kSub : len);
  partial = (ent.y & kPartialBit) != 0;
}

// Mask data of a key for a partial sub-tile: its tracks, or (lo, hi, 0, 0)
// when the entry marks key intervals.
__device__ inline int4 key_mask_data(const int4* ktracks, const int2* kint, int64_t row, bool interval) {
  if (interval) {
    const int2 iv = kint[row];
    return make_int4(iv.x, iv.y, 0, 0);
  }
  return ktracks[row];
}

// lo <= x < hi as one unsigned compare (x: a query's token index, -1 on pad
// rows; 0 <= lo < hi <= 2^30).
__device__ inline bool in_interval(int32_t x, int32_t lo, int32_t hi) {
  return (uint32_t)(x - lo) < (uint32_t)(hi - lo);
}

}  // namespace dev
}  // namespace bsm
