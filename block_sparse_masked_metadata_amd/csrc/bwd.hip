// Backward step kernels: one ring step of the masked attention backward,
// run against the FINAL log-sum-exp (MARBLE, "exact sequence parallelism for
// packed multimodal masks", section 03 "Exact ring attention accumulation":
// each step runs the attention backward against the final LSE, an fp32 dQ
// accumulator is carried across steps and each key shard's fp32 dK/dV
// accumulator travels with the shard).
//
// For a legal pair (i, j) of the step, with s_ij = scale * q_i . k_j:
//   P_ij = exp(s_ij - LSE_i),  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i)
//   dQ_i += scale * dS_ij k_j,  dK_j += scale * dS_ij q_i,  dV_j += P_ij dO_i
// (D_i = dO_i . O_i from the prep kernel).  Two deterministic kernels:
//   dq   : one workgroup per (query tile, query head), walking the tile's row
//          list in 64-key sub-tiles (the next one loaded direct-to-LDS into
//          the other buffer set while one is used);
//          S^T and dP^T put one query per lane, so LSE_i and D_i are lane
//          scalars; dQ^T += K^T dS^T reads K^T with the LDS transpose read.
//   dkdv : one workgroup per (key tile, key/value head), walking the tile's
//          column list for every query head of the group in 64-query
//          sub-tiles; S and dP put one key per lane; dV^T += dO^T P and
//          dK^T += Q^T dS read dO^T and Q^T with the LDS transpose read.  8
//          waves: four key groups of 32 times the two 32-query halves of a
//          sub-tile (two waves per SIMD), K and V rows in LDS, both
//          accumulators in registers; the halves' sums meet at the end.

#include "tile_common.hpp"

namespace bsm {
namespace {

using namespace dev;

constexpr int kListCache = 512;  // list entries of an item kept in LDS at a time

// Entry e of an item's list through an LDS window of kListCache entries.
// Called by all threads at the same point right after a __syncthreads();
// reloads the window (with its own barrier) when e falls outside it.
__device__ inline int2 list_entry(int2* sEnt, int& base, const int2* entries, int4 it, int e, int tid,
                                 int nthreads) {
  if (e < base || e >= base + kListCache) {
    base = e - e % kListCache;
    for (int i = tid; i < kListCache && base + i < it.w; i += nthreads) sEnt[i] = entries[it.z + base + i];
    __syncthreads();
  }
  return sEnt[e - base];
}

// s = A_rows(tileA) . b1 and dp = dp0 + A_rows(tileB) . b2 over the 128
// channels: the lane's row of two staged tiles (its 16-byte operands at the
// per-lane byte offsets ao[kk]) against two register operands, with the LDS
// operand reads issued 4 at a time ahead of their MFMAs.
__device__ inline void two_products(f32x16& s, f32x16& dp, const char* ta, const char* tb, const uint32_t (&ao)[8],
                                    const bf16x8 (&b1)[8], const bf16x8 (&b2)[8], float dp0) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = 0.f;
    dp[r] = dp0;
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    bf16x8 x[2], y[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      x[k] = as_bf16x8(*(const uint4*)(ta + ao[2 * g + k]));
      y[k] = as_bf16x8(*(const uint4*)(tb + ao[2 * g + k]));
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then 4 MFMAs
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      s = mfma(x[k], b1[2 * g + k], s);
      dp = mfma(y[k], b2[2 * g + k], dp);
    }
  }
}

// The same two products with both B operands read from staged tiles too
// (row `krow` of tiles tk and tv, the unit's K and V rows in LDS) and dp
// started from dp0.
__device__ inline void two_products_lds(f32x16& s, f32x16& dp, const char* ta, const char* tb, int row,
                                        const char* tk, const char* tv, int krow, int hi, const f32x16& dp0) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = 0.f;
    dp[r] = dp0[r];
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 x = row_operand(ta, row, kk, hi), y = row_operand(tb, row, kk, hi);
    const bf16x8 b1 = row_operand(tk, krow, kk, hi), b2 = row_operand(tv, krow, kk, hi);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // then 2 MFMAs
    s = mfma(x, b1, s);
    dp = mfma(y, b2, dp);
  }
}

// The same two products over per-lane byte offsets inside the staged tiles:
// ta/tb at ao[kk], tk/tv at ko[kk] (channels [16 kk + 8 hi, +8) of the rows).
__device__ inline void two_products_off(f32x16& s, f32x16& dp, const char* ta, const char* tb, const uint32_t (&ao)[8],
                                        const char* tk, const char* tv, const uint32_t (&ko)[8], const f32x16& dp0) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = 0.f;
    dp[r] = dp0[r];
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 x = as_bf16x8(*(const uint4*)(ta + ao[kk])), y = as_bf16x8(*(const uint4*)(tb + ao[kk]));
    const bf16x8 b1 = as_bf16x8(*(const uint4*)(tk + ko[kk])), b2 = as_bf16x8(*(const uint4*)(tv + ko[kk]));
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // then 2 MFMAs
    s = mfma(x, b1, s);
    dp = mfma(y, b2, dp);
  }
}

constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3: 32-bit data format, untyped loads
typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS copy of one 64-row sub-tile of K or V (one KV head) into the
// tile_slot layout: wave w issues 4 buffer loads of 16 B per lane, load i
// filling rows 16i + 4w .. +3 (1 KiB, lane l at byte 16 l).  Row r = 16i +
// 4w + l/16 has r % 4 = l/16 and (r / 4) % 4 = w, so the slot-to-chunk map,
// and with it each lane's source offset `voff`, is the same for every load.
// The record count ends at the sub-tile's last valid row, so rows past `len`
// arrive as zeros.  Both values are uniform; readfirstlane keeps them in
// scalar registers (one in a vector register costs a waterfall loop).  Byte
// offsets stay below 2^32 (a key buffer holds fewer than 2^32 bytes).
__device__ inline void dma_tile(const char* base, char* lds, int64_t r0, int len, uint32_t row_bytes, uint32_t voff,
                                int wave) {
  const int nrec = __builtin_amdgcn_readfirstlane((int)((uint32_t)(r0 + len) * row_bytes));
  const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)r0 * row_bytes));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nrec, kBufferFlags);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + 4096 * i + 1024 * wave), 16, voff,
                                             so + 16u * i * row_bytes, 0, 0);
}

// kDense: dense-call lists (entries carry a relation and query rows; the
// staged key data is the key's position, 2^31 - 1 past the valid rows).
// K and V sub-tiles reach LDS by direct-to-LDS loads into two buffers each
// (sub-tile n in set n % 2): the loads of sub-tile n + 1 fly while n
// computes, one workgroup barrier per sub-tile.
template <bool kDense>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char sK0[kSub * 256];
  __shared__ __attribute__((aligned(1024))) char sK1[kSub * 256];
  __shared__ __attribute__((aligned(1024))) char sV0[kSub * 256];
  __shared__ __attribute__((aligned(1024))) char sV1[kSub * 256];
  __shared__ int4 sKT0[kSub];
  __shared__ int4 sKT1[kSub];
  __shared__ int2 sEnt[kListCache];

  int32_t item, h;
  map_block((int32_t)blockIdx.x, a.nitems, a.hq, a.heads_per_xcd, item, h);
  if (item < 0) return;
  const int4 it = a.items[item];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t qrow = (int64_t)it.x * kTile + wave * 32 + l32;
  const bool qvalid = qrow < a.rows;
  const int32_t kvh = h / (a.hq / a.hkv);
  const uint32_t row_bytes = (uint32_t)a.hkv * kHeadDim * 2u;
  const char* kbase = (const char*)(a.k + (int64_t)kvh * kHeadDim);
  const char* vbase = (const char*)(a.v + (int64_t)kvh * kHeadDim);
  const int nsub = 2 * it.w;
  // this lane's source chunk in each direct-to-LDS load (tile_slot layout)
  const int rw = 4 * wave + (lane >> 4);
  const uint32_t voff = (uint32_t)rw * row_bytes + 16u * (uint32_t)((lane & 15) ^ (4 * (lane >> 4) + wave));

  int list_base = 0;

  // prologue: the first sub-tile, Q, dO, the row scalars, the first key data
  // and the list window are all issued before anything uses a loaded value,
  // into registers that nothing else writes, so it takes one memory round
  // trip after the first list entry.  An invalid query row reads the tile's
  // first row (always present) and is replaced afterwards; its p is 0 through
  // the -inf LSE.
  int2 ent = a.entries[it.z];
  ent.x = __builtin_amdgcn_readfirstlane(ent.x);
  ent.y = __builtin_amdgcn_readfirstlane(ent.y);
  int64_t r0f;
  int lenf;
  bool partf;
  sub_bounds(ent, 0, r0f, lenf, partf);
  dma_tile(kbase, sK0, r0f, lenf, row_bytes, voff, wave);
  dma_tile(vbase, sV0, r0f, lenf, row_bytes, voff, wave);
  const int64_t qr = qvalid ? qrow : (int64_t)it.x * kTile;
  bf16x8 qf[8], df[8];
  {
    const int64_t off = (qr * a.hq + h) * kHeadDim + hi * 8;
    const unsigned short* qp = (const unsigned short*)a.q + off;
    const unsigned short* dp = (const unsigned short*)a.dout + off;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = as_bf16x8(*(const uint4*)(qp + kk * 16));
      df[kk] = as_bf16x8(*(const uint4*)(dp + kk * 16));
    }
  }
  const int64_t sidx = (int64_t)h * a.rows + qr;
  const float lse_raw = a.lse[sidx], dl_raw = a.delta[sidx];
  const int4 qt_raw = a.qtracks[qr];
  const int32_t qc_raw = a.qcoord[qr];
  const bool kload = partf && lenf > 0, kinterval = (ent.y & kIntervalBit) != 0;
  int4 kraw;  // an interval fills x and y only
  if (kload) {
    const int64_t kr = r0f + (tid < lenf ? tid : lenf - 1);
    if (kDense) {
      kraw.x = a.ktracks[kr].w;
    } else if (kinterval) {
      const int2 iv = a.kint[kr];
      kraw.x = iv.x;
      kraw.y = iv.y;
    } else {
      kraw = a.ktracks[kr];
    }
  }
  for (int i = tid; i < it.w && i < kListCache; i += 256) sEnt[i] = a.entries[it.z + i];
  const float nlse2 = qvalid ? -lse_raw * kLog2e : kNegInf;  // invalid rows: p = 0
  const float dl = qvalid ? dl_raw : 0.f;
  const int4 qt = query_tracks(qvalid ? qt_raw : make_int4(0, -1, -1, 0));
  const int32_t qc = qvalid ? qc_raw : -1;  // the query's token index (key-interval coordinate)
  int4 kt0 = make_int4(kDense ? INT32_MAX : -1, -1, -1, 0);  // keys past len: sample -1, empty range
  if (kload && tid < lenf) {
    if (kDense)
      kt0.x = kraw.x;
    else
      kt0 = kinterval ? make_int4(kraw.x, kraw.y, 0, 0) : kraw;
  }

  f32x16 acc[4];  // dQ^T[d = 32db + 8(r/4) + 4hi + r%4][query l32], unscaled
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  if (tid < kSub) sKT0[tid] = kt0;
  __builtin_amdgcn_s_waitcnt(0);  // no load is pending when the loop starts (direct-to-LDS ones included)
  __syncthreads();
  // Per-lane byte offsets of the loop's LDS reads inside a staged sub-tile,
  // the same for every sub-tile: the row reads of the lane's key (keys
  // 32 kc + l32 at +8192 kc) and the transposed reads (channels 32 db..,
  // rows r and r + 8 of a 16-key group; group 2 kc + hf at +4096 (2 kc + hf)).
  uint32_t kro[8], tro[4][2];
  {
    const TrLane tr(lane);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kro[kk] = (uint32_t)tile_slot(l32, 2 * kk + hi);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      tro[db][0] = (uint32_t)(tile_slot(tr.row0, 4 * db + tr.chunk) + tr.off8);
      tro[db][1] = (uint32_t)(tile_slot(tr.row0 + 8, 4 * db + tr.chunk) + tr.off8);
    }
  }

  // Sub-tile n from buffer set (sK, sV, sKT); the loads of n + 1 go to the
  // other set (nK, nV, nKT), which every wave finished with before the
  // barrier that precedes this call.
  auto step = [&](int n, const char* sK, const char* sV, const int4* sKT, char* nK, char* nV, int4* nKT) {
    int64_t r0;
    int len;
    bool partial;
    sub_bounds(ent, n, r0, len, partial);
    const bool interval = (ent.y & kIntervalBit) != 0;
    const int32_t ey = ent.y;
    const bool more = n + 1 < nsub;
    int4 kt_pf = make_int4(kDense ? INT32_MAX : -1, -1, -1, 0);  // keys past len: sample -1, empty range
    if (more) {
      if (n & 1) {
        ent = list_entry(sEnt, list_base, a.entries, it, (n + 1) >> 1, tid, 256);
        ent.x = __builtin_amdgcn_readfirstlane(ent.x);
        ent.y = __builtin_amdgcn_readfirstlane(ent.y);
      }
      int64_t nr0;
      int nlen;
      bool npart;
      sub_bounds(ent, n + 1, nr0, nlen, npart);
      if (npart && tid < nlen) {
        if (kDense)
          kt_pf.x = a.ktracks[nr0 + tid].w;
        else
          kt_pf = key_mask_data(a.ktracks, a.kint, nr0 + tid, (ent.y & kIntervalBit) != 0);
      }
      dma_tile(kbase, nK, nr0, nlen, row_bytes, voff, wave);
      dma_tile(vbase, nV, nr0, nlen, row_bytes, voff, wave);
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      f32x16 s, dp;
      two_products(s, dp, sK + 8192 * kc, sV + 8192 * kc, kro, qf, df, -dl);  // dp = dP - delta
      // s[r] = S[query l32][key 32kc + 8(r/4) + 4hi + r%4]
      if (kDense) {
        if (partial) {
          int32_t dlo;
          uint32_t dspan;
          dense_range(ey, wave * 32 + l32, qt.w, a.window, dlo, dspan);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kc * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            s[r] = (uint32_t)sKT[key].x - (uint32_t)dlo < dspan ? s[r] : kNegInf;
          }
        }
      } else if (partial && interval) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kc * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const int2 iv = *(const int2*)&sKT[key];
          s[r] = in_interval(qc, iv.x, iv.y) ? s[r] : kNegInf;
        }
      } else if (partial) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kc * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          s[r] = legal(qt, sKT[key], a.window) ? s[r] : kNegInf;  // keys past len: sample -1
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, nlse2));
        dp[r] = p * dp[r];
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8 dsb;
#pragma unroll
        for (int i = 0; i < 8; ++i) dsb[i] = (__bf16)dp[8 * hf + i];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const char* t = sK + 4096 * (2 * kc + hf);
          acc[db] = mfma(lds_tr8(t + tro[db][0], t + tro[db][1]), dsb, acc[db]);
        }
      }
    }
    if (more && tid < kSub) nKT[tid] = kt_pf;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of sub-tile n + 1 have landed
    __syncthreads();  // sub-tile n + 1 is in LDS; every wave is done with sub-tile n
  };
  for (int n = 0; n < nsub; n += 2) {
    step(n, sK0, sV0, sKT0, sK1, sV1, sKT1);
    step(n + 1, sK1, sV1, sKT1, sK0, sV0, sKT0);
  }

  if (!qvalid) return;
  float* out = a.dq + (qrow * a.hq + h) * kHeadDim;
  const bool first = (it.y & kFirst) != 0;
  // every running value is read before the first store (interleaved, each
  // load waits for the store before it: one memory round trip per float4)
  float4 o4[16];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o4[4 * db + i] = first ? make_float4(0.f, 0.f, 0.f, 0.f) : *(const float4*)(out + db * 32 + i * 8 + hi * 4);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 x = o4[4 * db + i];
      x.x += a.scale * acc[db][4 * i + 0];
      x.y += a.scale * acc[db][4 * i + 1];
      x.z += a.scale * acc[db][4 * i + 2];
      x.w += a.scale * acc[db][4 * i + 3];
      *(float4*)(out + db * 32 + i * 8 + hi * 4) = x;
    }
}

// Row scalars and tracks of one 64-row query sub-tile, staged with Q and dO:
// threads 0..63 carry -LSE*log2(e), 64..127 delta, 128..191 the query tracks.
struct RowStage {
  float v;  // LSE (wave 0) or delta (wave 1), raw
  int4 t;
};

// dK/dV workgroups: 8 waves over one (key tile, kv head) unit.  Waves w and
// w + 4 hold the same 32 keys (w % 4) and take the two 32-query halves of
// every staged query sub-tile, so two waves share each SIMD and one's vector
// work runs beside the other's products.  The unit's K and V rows sit in LDS
// (the B operands of S and dP), which leaves each wave its two fp32
// accumulators and one half's products in 256 registers.  After the list the
// two halves' partial sums meet through LDS: waves 0-3 finish dK, waves 4-7 dV.
constexpr int kDkdvThreads = 512;

// kDense: dense-call column lists (entries carry a relation and the key rows
// of the tile they apply to).
template <bool kDense>
__global__ __launch_bounds__(kDkdvThreads, 2) void bwd_dkdv_kernel(const BwdArgs a) {
  // two buffer sets: sub-tile m computes from set m % 2 while m + 1 is
  // loaded into the other, one barrier per sub-tile.  Q and dO reach LDS by
  // direct-to-LDS loads (each set its own array, so the compiler tells a load
  // into one from reads of the other); the row scalars go through registers.
  __shared__ __attribute__((aligned(4096))) char sQ0[kSub * 256];
  __shared__ __attribute__((aligned(4096))) char sQ1[kSub * 256];
  __shared__ __attribute__((aligned(4096))) char sO0[kSub * 256];
  __shared__ __attribute__((aligned(4096))) char sO1[kSub * 256];
  __shared__ __attribute__((aligned(1024))) char sK[kTile * 256];  // the unit's K rows (two 64-row sub-tiles)
  __shared__ __attribute__((aligned(1024))) char sV[kTile * 256];
  __shared__ __attribute__((aligned(16))) float sL[2][kSub];
  __shared__ __attribute__((aligned(16))) float sD[2][kSub];
  __shared__ int4 sQT[2][kSub];
  __shared__ int2 sEnt[kListCache];

  int32_t unit, g;
  map_block((int32_t)blockIdx.x, a.nitems, a.hkv, a.heads_per_xcd, unit, g);
  if (unit < 0) return;
  // the unit's sub-tiles [n0, n0 + nsub) of its item's column list, for every
  // query head of the group (a split list cuts long lists into such ranges)
  const int4 wk = a.work ? a.work[unit] : make_int4(unit, 0, -1, -1);
  const int4 it = a.items[wk.x];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3, qh = wave >> 2;  // key group (32 keys), query half of each sub-tile
  const int l32 = lane & 31, hi = lane >> 5;
  const int krel = kw * 32 + l32;            // the lane's key within the tile
  const int64_t key = (int64_t)it.x + krel;  // it.x: the tile's first key row
  const bool kvalid = krel < key_rows(it.y);
  const int32_t grp = a.hq / a.hkv;
  const uint32_t row_bytes = (uint32_t)a.hq * kHeadDim * 2u;
  const int n0 = wk.y;
  const int nsub = (wk.z < 0 ? 2 * it.w : wk.z) - n0;
  const int total = grp * nsub;  // (query head of the group, sub-tile) pairs

  int list_base = 0;
  // every key of the tile has a key interval: partial pairs test the query's
  // token index against it (staged in place of the query tracks)
  const bool kin = (it.y & kKeyInterval) != 0;

  // direct-to-LDS loads (tile_slot layout; waves 0-3 issue them): lane l
  // of wave w reads row 4 w + l / 16 of each group of 16, chunk (l % 16) ^
  // f(row), as dma_tile lays them out
  // Load (head g*grp + m/nsub, sub-tile m%nsub): Q and dO into buffer set
  // (dq, ddo) by direct-to-LDS loads, the row scalars into registers.
  RowStage rs;
  int2 ent;
  bool cur_partial = false, nxt_partial = false;
  int cur_len = 0, nxt_len = 0;
  int32_t cur_ey = 0, nxt_ey = 0;  // entry words (dense-call relation and key rows)
  auto fetch = [&](int m, int2 e2, char* dq_, char* ddo) {
    const int32_t h = g * grp + m / nsub;
    int64_t r0;
    sub_bounds(e2, n0 + m % nsub, r0, nxt_len, nxt_partial);
    nxt_ey = e2.y;
    // Wave 0 loads the LSE rows, wave 1 the delta rows, wave 2 the query
    // tracks (partial sub-tiles only), raw into registers set beforehand:
    // nothing computes on a loaded value before stage(), and no register
    // is written after a load into it is issued, so no wave waits here
    // before issuing the Q/dO loads.
    const int row = lane;  // the wave's 64 lanes cover the sub-tile's rows
    rs.v = 0.f;
    rs.t = make_int4(-2, -1, -1, -1);  // rows past len: no sample, no position
    if (wave < 2 && row < nxt_len) rs.v = (wave == 0 ? a.lse : a.delta)[(int64_t)h * a.rows + r0 + row];
    if (wave == 2 && nxt_partial && row < nxt_len) {
      if (kin)
        rs.t.w = a.qcoord[r0 + row];
      else
        rs.t = a.qtracks[r0 + row];
    }
    if (wave < 4) {
      const uint32_t voff = (uint32_t)(4 * kw + (lane >> 4)) * row_bytes + 16u * (uint32_t)((lane & 15) ^ (4 * (lane >> 4) + kw));
      dma_tile((const char*)(a.q + (int64_t)h * kHeadDim), dq_, r0, nxt_len, row_bytes, voff, wave);
      dma_tile((const char*)(a.dout + (int64_t)h * kHeadDim), ddo, r0, nxt_len, row_bytes, voff, wave);
    }
  };
  auto stage = [&](int buf) {
    if (wave == 0) sL[buf][lane] = lane < nxt_len ? -rs.v * kLog2e : kNegInf;
    else if (wave == 1) sD[buf][lane] = -rs.v;  // the dP products start from -delta
    else if (wave == 2) sQT[buf][lane] = query_tracks(rs.t);
  };

  // the unit's K/V rows depend on nothing loaded: issue them before the
  // list entry and the first query sub-tile that depends on it (rows past
  // the tile's valid keys arrive as zeros)
  if (wave < 4) {
    const uint32_t krow_bytes = (uint32_t)a.hkv * kHeadDim * 2u;
    const uint32_t kvoff = (uint32_t)(4 * kw + (lane >> 4)) * krow_bytes + 16u * (uint32_t)((lane & 15) ^ (4 * (lane >> 4) + kw));
    const int krows = key_rows(it.y);
    const char* kb = (const char*)(a.k + (int64_t)g * kHeadDim);
    const char* vb = (const char*)(a.v + (int64_t)g * kHeadDim);
    const int len0 = krows < kSub ? krows : kSub, len1 = krows - len0;
    dma_tile(kb, sK, it.x, len0, krow_bytes, kvoff, wave);
    dma_tile(kb, sK + kSub * 256, it.x + kSub, len1, krow_bytes, kvoff, wave);
    dma_tile(vb, sV, it.x, len0, krow_bytes, kvoff, wave);
    dma_tile(vb, sV + kSub * 256, it.x + kSub, len1, krow_bytes, kvoff, wave);
  }
  // this lane's key: its tracks, or its key interval when every key of the
  // tile has one (kKeyInterval); invalid keys admit no query
  // Loaded raw with no value written into these registers afterwards; an
  // invalid key reads the tile's first row (always present) and is replaced
  // once every prologue load has landed.
  const int64_t krow = kvalid ? key : (int64_t)it.x;
  int4 kraw;
  if (kin) {
    kraw.z = 0;
    kraw.w = 0;
    const int2 iv = a.kint[krow];
    kraw.x = iv.x;
    kraw.y = iv.y;
  } else {
    kraw = a.ktracks[krow];
  }
  ent = a.entries[it.z + (n0 >> 1)];
  ent.x = __builtin_amdgcn_readfirstlane(ent.x);
  ent.y = __builtin_amdgcn_readfirstlane(ent.y);
  fetch(0, ent, sQ0, sO0);
  for (int i = tid; i < it.w && i < kListCache; i += kDkdvThreads) sEnt[i] = a.entries[it.z + i];
  const int4 kt = kvalid ? kraw : make_int4(-1, -1, -1, 0);
  f32x16 dk[4], dv[4];  // dK^T / dV^T[d = 32db + 8(r/4) + 4hi + r%4][key]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }
  stage(0);
  cur_len = nxt_len;
  cur_partial = nxt_partial;
  cur_ey = nxt_ey;
  __builtin_amdgcn_s_waitcnt(0);  // no load is pending when the loop starts (direct-to-LDS ones included)
  __syncthreads();
  // Per-lane byte offsets of the loop's LDS reads inside a staged tile, the
  // same for every sub-tile: the transposed reads of the wave's query rows
  // (channels 32 db.., rows r and r + 8; the second 16-row half at +4096),
  // and the row reads of its query rows and of its keys.
  uint32_t tro[4][2], qro[8], kro[8];
  {
    const TrLane tr(lane);
    const int r = 32 * qh + tr.row0;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      tro[db][0] = (uint32_t)(tile_slot(r, 4 * db + tr.chunk) + tr.off8);
      tro[db][1] = (uint32_t)(tile_slot(r + 8, 4 * db + tr.chunk) + tr.off8);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qro[kk] = (uint32_t)tile_slot(32 * qh + l32, 2 * kk + hi);
      kro[kk] = (uint32_t)tile_slot(krel, 2 * kk + hi);
    }
  }

  // P = exp2(S * scale*log2(e) - LSE*log2(e)) and dS = P (dP - delta) for the
  // 32 queries [q0, q0+32) of the staged sub-tile, as bf16 MFMA B operands
  // (lane: key; register r: query q0 + 8(r/4) + 4hi + r%4); dp arrives as
  // dP - delta (its products start from -delta).  On partial sub-tiles
  // illegal pairs get P = 0; rows past len carry sample -2.
  auto p_and_ds = [&](f32x16& s, f32x16& dp, bf16x8 (&pb)[2], bf16x8 (&dsb)[2], int q0, bool partial,
                      const float* sL, const int4* sQT, int32_t ey) {
    if (kDense) {
      if (partial) {
        int32_t dlo;
        uint32_t dspan;
        dense_key_range(ey, krel, kt.w, a.window, dlo, dspan);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + 8 * (r >> 2) + 4 * hi + (r & 3);
          s[r] = (uint32_t)sQT[qi].w - (uint32_t)dlo < dspan ? s[r] : kNegInf;
        }
      }
    } else if (partial && kin) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[r] = in_interval(sQT[qi].w, kt.x, kt.y) ? s[r] : kNegInf;
      }
    } else if (partial) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[r] = legal(sQT[qi], kt, a.window) ? s[r] : kNegInf;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q4 = q0 + 8 * i + 4 * hi;
      const float4 l4 = *(const float4*)(sL + q4);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 4 * i + c;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, lv[c]));
        s[r] = p;
        dp[r] = p * dp[r];
      }
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pb[hf][i] = (__bf16)s[8 * hf + i];
        dsb[hf][i] = (__bf16)dp[8 * hf + i];
      }
  };
  // dV^T += dO^T P^T and dK^T += Q^T dS^T over the queries [q0, q0+32).
  auto accumulate = [&](const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2], int q0, const char* sQ, const char* sO) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dv[db] = mfma(lds_tr8(sO + 4096 * hf + tro[db][0], sO + 4096 * hf + tro[db][1]), pb[hf], dv[db]);
        dk[db] = mfma(lds_tr8(sQ + 4096 * hf + tro[db][0], sQ + 4096 * hf + tro[db][1]), dsb[hf], dk[db]);
      }
  };

  // Sub-tile m computes from set (cq, co, cb); the loads of m + 1 go to the
  // other set (nq, no), which every wave finished with before the barrier
  // that precedes this call.
  auto step = [&](int m, const char* cq, const char* co, int cb, char* nq, char* no) {
    const bool partial = cur_partial;
    const int32_t ey = cur_ey;
    const bool more = m + 1 < total;
    if (more) {
      // next sub-tile n0 + (m + 1) % nsub: a new list entry at an even
      // sub-tile, and at the start of the next head's range
      const int r1 = (m + 1) % nsub, n1 = n0 + r1;
      if ((n1 & 1) == 0 || r1 == 0) {
        ent = list_entry(sEnt, list_base, a.entries, it, n1 >> 1, tid, kDkdvThreads);
        ent.x = __builtin_amdgcn_readfirstlane(ent.x);
        ent.y = __builtin_amdgcn_readfirstlane(ent.y);
      }
      fetch(m + 1, ent, nq, no);
    }
    // this wave's 32-query half of the sub-tile against its 32 keys
    const int q0 = 32 * qh;
    f32x16 s0, dp0, nd;  // nd: -delta of the lane's 16 query rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 d4 = *(const float4*)(sD[cb] + q0 + 8 * i + 4 * hi);
      nd[4 * i + 0] = d4.x;
      nd[4 * i + 1] = d4.y;
      nd[4 * i + 2] = d4.z;
      nd[4 * i + 3] = d4.w;
    }
    bf16x8 pb0[2], ds0[2];
    // the MFMA blocks run at raised wave priority: the SIMD's arbiter issues
    // them ahead of the other wave's vector work
    __builtin_amdgcn_s_setprio(1);
    two_products_off(s0, dp0, cq, co, qro, sK, sV, kro, nd);  // dp0 = dP - delta
    __builtin_amdgcn_s_setprio(0);
    p_and_ds(s0, dp0, pb0, ds0, q0, partial, sL[cb], sQT[cb], ey);
    __builtin_amdgcn_s_setprio(1);
    accumulate(pb0, ds0, q0, cq, co);
    __builtin_amdgcn_s_setprio(0);
    if (more) {
      stage(cb ^ 1);  // the other set was last read in iteration m - 1
      cur_len = nxt_len;
      cur_partial = nxt_partial;
      cur_ey = nxt_ey;
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of sub-tile m + 1 have landed
    __syncthreads();  // sub-tile m + 1 is in LDS; every wave is done with m
  };
  int m = 0;
  for (; m + 1 < total; m += 2) {
    step(m, sQ0, sO0, 0, sQ1, sO1);
    step(m + 1, sQ1, sO1, 1, sQ0, sO0);
  }
  if (m < total) step(m, sQ0, sO0, 0, sQ1, sO1);

  // The two query halves' partial sums meet through LDS, free after the
  // loop's last barrier: waves 4-7 leave their dK partials, waves 0-3 their
  // dV partials (16 KiB a wave, lane l's float4 number n at 1024 n + 16 l),
  // and each side adds the other's: waves 0-3 then hold dK, waves 4-7 dV.
  {
    char* xk = kw == 0 ? sQ0 : kw == 1 ? sQ1 : kw == 2 ? sO0 : sO1;
    char* xv = (kw < 2 ? sK : sV) + (kw & 1) * 16384;
    char* mine = qh ? xk : xv;
    const f32x16* give = qh ? dk : dv;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(float4*)(mine + 1024 * (4 * db + i) + 16 * lane) =
            make_float4(give[db][4 * i], give[db][4 * i + 1], give[db][4 * i + 2], give[db][4 * i + 3]);
    __syncthreads();
    const char* theirs = qh ? xv : xk;
    f32x16* keep = qh ? dv : dk;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 o4 = *(const float4*)(theirs + 1024 * (4 * db + i) + 16 * lane);
        keep[db][4 * i + 0] += o4.x;
        keep[db][4 * i + 1] += o4.y;
        keep[db][4 * i + 2] += o4.z;
        keep[db][4 * i + 3] += o4.w;
      }
  }
  if (!kvalid) return;
  // waves 0-3: dK, scaled; waves 4-7: dV
  const f32x16* res = qh ? dv : dk;
  const float mul = qh ? 1.f : a.scale;
  if (wk.w >= 0) {
    // a split unit: its partial goes to its workspace slot (dK, then dV)
    float* wp = a.ws + ((int64_t)wk.w * a.hkv + g) * (2 * kTile * kHeadDim) + qh * (kTile * kHeadDim) +
                krel * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = db * 32 + i * 8 + hi * 4;
        *(float4*)(wp + c) = make_float4(mul * res[db][4 * i], mul * res[db][4 * i + 1],
                                         mul * res[db][4 * i + 2], mul * res[db][4 * i + 3]);
      }
    return;
  }
  // every running value is read before the first store (one memory round
  // trip), then each is added to and stored
  float* run = (qh ? a.dv : a.dk) + (key * a.hkv + g) * kHeadDim;
  float4 r4[16];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) r4[4 * db + i] = *(const float4*)(run + db * 32 + i * 8 + hi * 4);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 x = r4[4 * db + i];
      x.x += mul * res[db][4 * i + 0];
      x.y += mul * res[db][4 * i + 1];
      x.z += mul * res[db][4 * i + 2];
      x.w += mul * res[db][4 * i + 3];
      *(float4*)(run + db * 32 + i * 8 + hi * 4) = x;
    }
}

// One workgroup per (reduce entry, kv head): dk/dv of the entry's key tile
// += its workspace slots in slot order (deterministic), one float4 per
// thread and step.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const BwdArgs a) {
  const int32_t e = (int32_t)blockIdx.x / a.hkv, g = (int32_t)blockIdx.x % a.hkv;
  const int4 rd = a.reduce[e];
  // kU float4 per thread per round, all read before any store: dk and dv may
  // alias as far as the compiler knows, so a load placed after a store waits
  // for a memory round trip of its own.  Each element still adds its slots in
  // slot order.
  constexpr int kN = kTile * kHeadDim / 4, kU = 4;
  static_assert(kN % (256 * kU) == 0, "rounds cover the key tile exactly");
  for (int i0 = threadIdx.x; i0 < kN; i0 += 256 * kU) {
    float4 k4[kU], v4[kU];
    int64_t off[kU];
    bool ok[kU];
    int rc[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + 256 * u, row = i / (kHeadDim / 4), c = (i % (kHeadDim / 4)) * 4;
      const int64_t key = (int64_t)rd.x + row;
      ok[u] = row < rd.w;
      off[u] = (key * a.hkv + g) * kHeadDim + c;
      rc[u] = row * kHeadDim + c;
      k4[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      v4[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok[u]) {
        k4[u] = *(const float4*)(a.dk + off[u]);
        v4[u] = *(const float4*)(a.dv + off[u]);
      }
    }
    for (int sl = rd.y; sl < rd.y + rd.z; ++sl) {
      const float* wp = a.ws + ((int64_t)sl * a.hkv + g) * (2 * kTile * kHeadDim);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float4 pk = *(const float4*)(wp + rc[u]);
        const float4 pv = *(const float4*)(wp + kTile * kHeadDim + rc[u]);
        k4[u].x += pk.x;
        k4[u].y += pk.y;
        k4[u].z += pk.z;
        k4[u].w += pk.w;
        v4[u].x += pv.x;
        v4[u].y += pv.y;
        v4[u].z += pv.z;
        v4[u].w += pv.w;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (ok[u]) {
        *(float4*)(a.dk + off[u]) = k4[u];
        *(float4*)(a.dv + off[u]) = v4[u];
      }
  }
}

// The sparse fetch's way back (MARBLE section 04: the fetched blocks' dK and
// dV return with the inverse all-to-all and are accumulated in fp32 by their
// owner): one thread per float4 of a compact row and kv head.  Each shard row
// appears at most once in the compact buffer, so no two threads add into one
// element.
__global__ __launch_bounds__(256) void fetch_accumulate_kernel(const FetchAccArgs a) {
  const int64_t quads = (int64_t)a.hkv * (kHeadDim / 4);
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= a.rows * quads) return;
  const int64_t c = g / quads, e = (g % quads) * 4;
  const int32_t src = a.src[c];
  if (src < 0) return;
  const int64_t from = c * a.hkv * kHeadDim + e, to = (int64_t)src * a.hkv * kHeadDim + e;
  const float4 k = *(const float4*)(a.dk_fetch + from), v = *(const float4*)(a.dv_fetch + from);
  float4 x = *(const float4*)(a.dk + to), y = *(const float4*)(a.dv + to);
  x.x += k.x;
  x.y += k.y;
  x.z += k.z;
  x.w += k.w;
  y.x += v.x;
  y.y += v.y;
  y.z += v.z;
  y.w += v.w;
  *(float4*)(a.dk + to) = x;
  *(float4*)(a.dv + to) = y;
}

}  // namespace

hipError_t launch_fetch_accumulate(const FetchAccArgs& a, hipStream_t stream) {
  const int64_t threads = a.rows * a.hkv * (kHeadDim / 4);
  if (threads <= 0) return hipSuccess;
  hipLaunchKernelGGL(fetch_accumulate_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.nreduce * a.hkv;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.nitems * a.hq;
  if (blocks <= 0) return hipSuccess;
  if (a.dense)
    hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.nitems * a.hkv;
  if (blocks <= 0) return hipSuccess;
  if (a.dense)
    hipLaunchKernelGGL(bwd_dkdv_kernel<true>, dim3((unsigned)blocks), dim3(kDkdvThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dkdv_kernel<false>, dim3((unsigned)blocks), dim3(kDkdvThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsm
