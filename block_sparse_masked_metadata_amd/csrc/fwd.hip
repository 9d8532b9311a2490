// Forward step kernel: one ring step (or the merged single pass) of exact
// block-sparse masked attention with the fp32 online-softmax state carried in
// HBM between steps.
//
// MARBLE ("exact sequence parallelism for packed multimodal masks"),
// section 03 "Exact ring attention accumulation": each step is the
// FlashAttention loop over a different set of key blocks; the fp32
// accumulator, row max m and row sum l live in HBM between calls, every call
// but the first starts from the stored state, and only the last call
// normalizes, writes LSE and rounds O to bf16.  Section 03 "Block
// classification": a key tile tagged full skips the mask, a partial one runs
// the mask predicate of section 01 on every element.
//
// Work decomposition: one workgroup of 4 waves per (query tile, query head);
// wave w owns query rows [32w, 32w+32) of the tile.  Per listed key tile:
//   1. the 128x128 K and V tiles are staged in LDS (row-major, padded rows);
//   2. S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K from LDS is the A operand,
//      Q (kept in registers for the whole item) the B operand, so the result
//      puts one query per lane (lane l and l^32 share query l%32, each holding
//      half of the tile's keys);
//   3. the online softmax is then mostly lane-local (one cross-lane exchange
//      for the row max and one for the row sum), in base-2 units with
//      scale*log2(e) folded into one multiply;
//   4. O^T += V^T P^T on MFMA: P (bf16) is the B operand straight from the
//      registers of step 3, with the 16 key slots of each MFMA permuted to
//      match the accumulator layout; V^T is read from the row-major V tile
//      with the gfx950 LDS transpose read (ds_read_b64_tr_b16) at the same
//      permutation.  The output accumulator again holds one query per lane,
//      so the rescale by exp2(m_old - m_new) is a per-lane scalar.

#include "tile_common.hpp"

namespace bsm {
namespace {

using dev::bf16x8;
using dev::f32x16;
using dev::kNegInf;
using dev::kLn2;
using dev::kSub;
using dev::as_bf16x8;
using dev::lds_tr8;
using dev::legal;
using dev::query_tracks;
using dev::map_block;

// ---- LDS sub-tiles: 64 key rows x 256 B, unpadded, 16-byte chunks XOR-swizzled ----
// K: chunk c of row r sits in slot c ^ (r & 15), so the MFMA A-operand reads
//    (one chunk of 16 consecutive rows per 16 lanes) hit 16 distinct slots.
// V: chunk c of row r sits in slot c ^ 4(r & 3), so each transpose read
//    (4 rows x 4 chunks per 32 lanes) hits 16 distinct slots.
__device__ inline int k_slot(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
__device__ inline int v_slot(int r, int c) { return r * 256 + ((c ^ ((r & 3) << 2)) << 4); }

constexpr int kListCache = 512;      // list entries of an item kept in LDS
constexpr float kSumCap = 4096.0f;   // a lane sum below 2^12 keeps every p below 2^12
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3: 32-bit data format, untyped loads

// One sub-tile of K, V (and key tracks) staged through registers: thread t
// holds chunk t%16 of rows t/16 + 16i (i = 0..3), so every 16 lanes read one
// 256-byte row contiguously.  Rows past `len` are zero.
struct SubTile {
  uint4 k[4], v[4];
  int4 kt;
};

// kbase/vbase: the head's element 0 of key row 0 (uniform).  k0 is uniform, so
// the row base of a full sub-tile and the strides of its 4 loads are scalar;
// `lane_off` = (t/16) * row_bytes + 16 (t%16) is loop-invariant.  Key-row byte
// offsets stay below 2^32 (a key buffer holds fewer than 2^32 bytes).
// On partial sub-tiles the key's mask data rides along: its tracks, or with
// `interval` its key interval (lo, hi) in the first two fields.  Keys past len
// keep (-1, -1, -1, 0): sample -1 and the empty range [-1, -1) admit no query.
// With kDense (dense-call lists) a partial sub-tile carries only the key's
// position, and keys past len take position 2^31 - 1, outside every range.
template <bool kDense>
__device__ inline void fetch_sub(SubTile& t, const char* kbase, const char* vbase,
                                 const int4* ktracks, const int2* kint, int32_t k0, int len, bool partial,
                                 bool interval, uint32_t row_bytes, uint32_t lane_off, int tid) {
  t.kt = make_int4(kDense ? INT32_MAX : -1, -1, -1, 0);
  if (partial && tid < len) {
    if (kDense) {
      t.kt.x = ktracks[k0 + tid].w;
    } else if (interval) {
      const int2 iv = kint[k0 + tid];
      t.kt = make_int4(iv.x, iv.y, 0, 0);
    } else {
      t.kt = ktracks[k0 + tid];
    }
  }
  const uint32_t r0 = (uint32_t)k0 * row_bytes;
  if (len == kSub) {
    // raw buffer loads: the uniform row offset rides in soffset and the
    // loop-invariant lane offset in voffset, so no per-load address
    // arithmetic.  The record count is the full 32-bit range: every byte
    // offset of a key buffer (under 4 GiB) is in range.
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, -1, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, -1, kBufferFlags);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ro = r0 + 16u * i * row_bytes;
      t.k[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off, ro, 0));
      t.v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, lane_off, ro, 0));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 4) + 16 * i;
      const uint32_t ro = r0 + 16u * i * row_bytes;
      t.k[i] = make_uint4(0, 0, 0, 0);
      t.v[i] = make_uint4(0, 0, 0, 0);
      if (row < len) {
        t.k[i] = *(const uint4*)(kbase + ro + lane_off);
        t.v[i] = *(const uint4*)(vbase + ro + lane_off);
      }
    }
  }
}

__device__ inline void store_sub(const SubTile& t, char* sK, char* sV, int4* sKT, int tid) {
  const int c = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 4) + 16 * i;
    *(uint4*)(sK + k_slot(row, c)) = t.k[i];
    *(uint4*)(sV + v_slot(row, c)) = t.v[i];
  }
  if (tid < kSub) sKT[tid] = t.kt;
}

// Sub-tile n of an item: half n%2 of list entry n/2.
__device__ inline void sub_bounds(const int2 ent, int n, int32_t& k0, int& len, bool& partial, bool& interval) {
  const int half = n & 1;
  const int klen = ent.y & kLenMask;
  k0 = ent.x + half * kSub;
  len = klen - half * kSub;
  len = len < 0 ? 0 : (len > kSub ? kSub : len);
  partial = (ent.y & kPartialBit) != 0;
  interval = (ent.y & kIntervalBit) != 0;
}

// S^T = K Q^T for one 64-key sub-tile: s[kb][r] = S[query l32][key 32kb + 8(r/4) + 4hi + r%4],
// operand reads issued 4 at a time ahead of their MFMAs; on partial sub-tiles
// illegal pairs (and keys past len) become -inf.
// With kDense, a partial sub-tile keeps the pairs whose key position lies in
// the range dense_range gives the lane's query for entry word `ey`.
template <bool kDense>
__device__ inline void scores(f32x16 (&s)[2], const char* sK, const bf16x8 (&qf)[8], const int4* sKT,
                              const int4 qt, int32_t qc, bool partial, bool interval, int32_t window, int l32,
                              int hi, int32_t ey, int row) {
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    const int row = kb * 32 + l32;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      bf16x8 kf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kf[kk] = as_bf16x8(*(const uint4*)(sK + k_slot(row, 2 * (4 * g + kk) + hi)));
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then 4 MFMAs
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[4 * g + kk], s[kb], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  if (kDense) {
    if (partial) {
      int32_t dlo;
      uint32_t dspan;
      dense_range(ey, row, qt.w, window, dlo, dspan);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          s[kb][r] = (uint32_t)sKT[key].x - (uint32_t)dlo < dspan ? s[kb][r] : kNegInf;
        }
    }
  } else if (partial && interval) {
    // Key intervals: legal iff lo <= qc < hi (qc: the query's token index),
    // one unsigned compare.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const int2 iv = *(const int2*)&sKT[key];
        s[kb][r] = (uint32_t)(qc - iv.x) < (uint32_t)(iv.y - iv.x) ? s[kb][r] : kNegInf;
      }
  } else if (partial) {
    // Keys past len carry sample -1 and fail the sample test.  Every lane of
    // a half-wave reads the same key track (an LDS broadcast); no branches.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[kb][r] = legal(qt, sKT[key], window) ? s[kb][r] : kNegInf;
      }
  }
}

// p = 2^(s * scale_log2 + nbase) in place; returns the lane's sum of p.
__device__ inline float exp_sum(f32x16 (&s)[2], float scale_log2, float nbase) {
  float ls = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], scale_log2, nbase));
      s[kb][r] = p;
      ls += p;
    }
  return ls;
}

template <bool kDense>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char sK[kSub * 256];
  __shared__ __attribute__((aligned(1024))) char sV[kSub * 256];
  __shared__ int4 sKT[kSub];
  __shared__ int2 sEnt[kListCache];

  int32_t item, h;
  map_block((int32_t)blockIdx.x, a.nitems, a.hq, a.heads_per_xcd, item, h);
  if (item < 0) return;
  // Prologue in two memory round trips: the item record and its first list
  // entry (scalar loads, side by side), then every other load at once: the
  // list, the first K/V sub-tile, Q, the query tracks and the state.
  int4 it = a.items[item];
  if (a.step_only) it.y = kFirst | kLast;  // this step's keys alone
  int2 ent = a.first[item];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // the item's list goes to LDS in chunks of kListCache entries, so the loop
  // never waits on a memory load for it (two entries per thread)
  const int nl = it.w < kListCache ? it.w : kListCache;
  int2 le0 = make_int2(0, 0), le1 = make_int2(0, 0);
  if (tid < nl) le0 = a.entries[it.z + tid];
  if (tid + 256 < nl) le1 = a.entries[it.z + 256 + tid];
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t q0 = (int64_t)it.x * kTile;
  const int64_t qi = wave * 32 + l32;
  const bool qvalid = q0 + qi < a.rows;
  const int64_t qrow = q0 + qi;
  const int32_t kvh = h / (a.hq / a.hkv);
  const uint32_t row_bytes = (uint32_t)a.hkv * kHeadDim * 2u;
  const char* kbase = (const char*)(a.k + (int64_t)kvh * kHeadDim);
  const char* vbase = (const char*)(a.v + (int64_t)kvh * kHeadDim);
  const int nsub = 2 * it.w;

  // prologue: fetch the first sub-tile, then Q and the state
  SubTile pf;
  const uint32_t lane_off = (uint32_t)(tid >> 4) * row_bytes + (uint32_t)(tid & 15) * 16u;
  ent.x = __builtin_amdgcn_readfirstlane(ent.x);
  ent.y = __builtin_amdgcn_readfirstlane(ent.y);
  {
    int32_t k0;
    int len;
    bool part, kin;
    sub_bounds(ent, 0, k0, len, part, kin);
    fetch_sub<kDense>(pf, kbase, vbase, a.ktracks, a.kint, k0, len, part, kin, row_bytes, lane_off, tid);
  }

  // Q^T as the B operand: lane holds query l32, channels [16kk + 8hi, +8).
  bf16x8 qf[8];
  {
    const unsigned short* qp = (const unsigned short*)a.q + (qrow * a.hq + h) * kHeadDim + hi * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = qvalid ? as_bf16x8(*(const uint4*)(qp + kk * 16)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  const int4 qt = query_tracks(qvalid ? a.qtracks[qrow] : make_int4(0, -1, -1, 0));
  const int32_t qc = qvalid ? a.qcoord[qrow] : -1;

  // Running state.  acc[db][r] = O^T[d = 32db + 8(r/4) + 4hi + r%4][query l32];
  // mref is the base-2 reference the accumulator and l are scaled against.
  f32x16 acc[4];
  float mref = kNegInf, lrun = 0.f;
  const int64_t sidx = (int64_t)h * a.rows + qrow;
  // this lane's part of the item's tile-blocked state (state_index): float4
  // number 4 db + i at op + 256 (4 db + i)
  float* op = a.oacc + ((int64_t)it.x * a.hq + h) * (kTile * kHeadDim) + wave * (32 * kHeadDim) + lane * 4;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  if (!(it.y & kFirst) && qvalid) {
    mref = a.m[sidx];
    lrun = a.l[sidx];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v4 = *(const float4*)(op + (db * 4 + i) * 256);
        acc[db][4 * i + 0] = v4.x;
        acc[db][4 * i + 1] = v4.y;
        acc[db][4 * i + 2] = v4.z;
        acc[db][4 * i + 3] = v4.w;
      }
  }
  if (tid < nl) sEnt[tid] = le0;
  if (tid + 256 < nl) sEnt[tid + 256] = le1;
  store_sub(pf, sK, sV, sKT, tid);
  // Drain every prologue load here, once: a register loaded before the loop
  // with a load still pending would make each iteration's first use of it
  // wait on the memory counter, i.e. on the in-flight prefetch as well.
  __builtin_amdgcn_s_waitcnt(0);

  // lane constants of the V transpose reads
  const int G = lane >> 4, jl = lane & 15;
  const int tr_row0 = 4 * (G >> 1) + (jl >> 2);
  const int tr_chunk = 2 * (G & 1) + ((jl & 3) >> 1);  // + 4 db
  const int tr_off8 = (jl & 1) * 8;

  for (int n = 0; n < nsub; ++n) {
    int32_t k0;
    int len;
    bool partial, interval;
    sub_bounds(ent, n, k0, len, partial, interval);
    const int32_t ey = ent.y;
    __syncthreads();  // sub-tile n is in LDS
    const bool more = n + 1 < nsub;
    if (more) {
      if (n & 1) {
        const int e1 = (n + 1) >> 1;
        if (e1 % kListCache == 0) {  // next chunk of the list (long lists only)
          for (int i = tid; i < kListCache && e1 + i < it.w; i += 256) sEnt[i] = a.entries[it.z + e1 + i];
          __syncthreads();
        }
        ent = sEnt[e1 % kListCache];
        ent.x = __builtin_amdgcn_readfirstlane(ent.x);
        ent.y = __builtin_amdgcn_readfirstlane(ent.y);
      }
      int32_t nk0;
      int nlen;
      bool npart, nkin;
      sub_bounds(ent, n + 1, nk0, nlen, npart, nkin);
      fetch_sub<kDense>(pf, kbase, vbase, a.ktracks, a.kint, nk0, nlen, npart, nkin, row_bytes, lane_off, tid);
    }

    f32x16 s[2];
    scores<kDense>(s, sK, qf, sKT, qt, qc, partial, interval, a.window, l32, hi, ey, (int)qi);

    // Online softmax in base-2 units against a lazily updated reference mref.
    // Common case: exponentiate against the current reference; every p stays
    // below 2^12 whenever the lane's sum does, and then nothing moves.  When a
    // row has no reference yet, or a lane's sum reaches 2^12 (the scores are
    // then recomputed: K is still in LDS), the wave takes the tile's row
    // maxima, moves the references and rescales O_acc and l.  Exact either
    // way: O_acc and l always share one reference.
    float ls;
    bool fast = !__any(mref == kNegInf);
    if (fast) {
      ls = exp_sum(s, a.scale_log2, -mref);
      if (__any(!(ls < kSumCap))) {
        fast = false;
        scores<kDense>(s, sK, qf, sKT, qt, qc, partial, interval, a.window, l32, hi, ey, (int)qi);
      }
    }
    if (!fast) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
      const float mnew = fmaxf(mref, mx);
      // 1 when this row's reference stays (also when it is still -inf), 0 from -inf
      const float alpha = mnew == mref ? 1.f : __builtin_amdgcn_exp2f(mref - mnew);
      lrun *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      mref = mnew;
      ls = exp_sum(s, a.scale_log2, mref == kNegInf ? 0.f : -mref);
    }
    ls += __shfl_xor(ls, 32);
    lrun += ls;
    bf16x8 pb[4];  // P^T as the B operand of 4 MFMAs of 16 keys each
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[t][i] = (__bf16)s[t >> 1][8 * (t & 1) + i];

    // O^T += V^T P^T, 16 keys per MFMA (the 4 operand reads of a key group first)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r0 = 16 * t + tr_row0;
      bf16x8 vf[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const char* p0 = sV + v_slot(r0, 4 * db + tr_chunk) + tr_off8;
        const char* p1 = sV + v_slot(r0 + 8, 4 * db + tr_chunk) + tr_off8;
        vf[db] = lds_tr8(p0, p1);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);  // 8 transpose reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);  // then 4 MFMAs
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pb[t], acc[db], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();  // every wave is done with sub-tile n
    if (more) store_sub(pf, sK, sV, sKT, tid);
  }

  if (!qvalid) return;
  if (!(it.y & kLast) || a.keep_state) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(float4*)(op + (db * 4 + i) * 256) =
            make_float4(acc[db][4 * i], acc[db][4 * i + 1], acc[db][4 * i + 2], acc[db][4 * i + 3]);
    if (hi == 0) {
      a.m[sidx] = mref;
      a.l[sidx] = lrun;
    }
  } else {
    // O = O_acc * (1 / l): one IEEE reciprocal per row instead of 64 IEEE
    // divisions per lane (one more fp32 rounding, far below the bf16 one),
    // then round to nearest even bf16.  A row with no legal key has l = 0 and
    // O_acc = 0, and writes zeros.
    const bool any = lrun > 0.f;
    const float rl = any ? 1.f / lrun : 0.f;
    unsigned short* out = (unsigned short*)a.o + (qrow * a.hq + h) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __bf16 b4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) b4[c] = (__bf16)(acc[db][4 * i + c] * rl);
        *(uint2*)(out + db * 32 + i * 8 + hi * 4) = __builtin_bit_cast(uint2, b4);
      }
    if (hi == 0) a.lse[sidx] = any ? (mref + __log2f(lrun)) * kLn2 : kNegInf;
  }
}

// ---- Accuracy controls (MARBLE section 03, "Exact ring attention
// accumulation", against the per-step merges it compares with) ----
// One step's partial result merged into a running one, per (row, head):
//   lse = log(e^lse_run + e^lse_s),  O = O_run e^(lse_run - lse) + O_s e^(lse_s - lse).
// Threads own 8 channels; 16 lanes cover one (row, head).  Rows the step did
// not reach (lse_s = -inf, or l = 0) keep the running values.
__device__ inline void merge_weights(float lr, float ls, float& wr, float& ws, float& lnew) {
  const float mx = fmaxf(lr, ls);
  const float er = expf(lr - mx), es = expf(ls - mx);  // lr = -inf -> er = 0
  lnew = mx + logf(er + es);
  wr = expf(lr - lnew);
  ws = expf(ls - lnew);
}

__global__ __launch_bounds__(256) void merge_bf16_kernel(int64_t pairs, int64_t rows, int32_t hq,
                                                         unsigned short* o_run, float* lse_run,
                                                         const unsigned short* o_s, const float* lse_s) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = gid >> 4;
  if (pair >= pairs) return;
  const int64_t row = pair / hq;
  const int32_t h = (int32_t)(pair % hq);
  const int64_t li = (int64_t)h * rows + row;
  const float ls = lse_s[li];
  if (ls == kNegInf) return;
  const float lr = lse_run[li];
  float wr, ws, lnew;
  merge_weights(lr, ls, wr, ws, lnew);
  const bf16x8 a8 = as_bf16x8(*(const uint4*)(o_run + gid * 8));
  const bf16x8 b8 = as_bf16x8(*(const uint4*)(o_s + gid * 8));
  bf16x8 r8;
#pragma unroll
  for (int i = 0; i < 8; ++i) r8[i] = (__bf16)((lr == kNegInf ? 0.f : wr * (float)a8[i]) + ws * (float)b8[i]);
  *(uint4*)(o_run + gid * 8) = __builtin_bit_cast(uint4, r8);
  if ((gid & 15) == 0) lse_run[li] = lnew;
}

// One workgroup per 32-row block of one (query tile, head) of the
// tile-blocked partial (4096 floats, one wave's rows in the forward): the
// block is read in its stored order, 16 bytes per thread, coalesced; each
// thread then updates the 4 channels of O_run that its float4 holds.  A
// row's merge weights are computed once, into LDS, and LSE_run is written
// only after every read of it.
__global__ __launch_bounds__(256) void merge_fp32_kernel(int64_t rows, int32_t hq, float* o_run, float* lse_run,
                                                         const float* acc_s, const float* m_s, const float* l_s,
                                                         unsigned short* o_bf16) {
  __shared__ float sw_r[32], sw_s[32], s_l[32], s_lnew[32];
  __shared__ int s_live[32];  // 0: row past the end, 1: merge, 2: not reached by this step
  __shared__ int s_fresh[32];  // no running value yet (LSE_run = -inf): O_run is ignored
  const int64_t blk = blockIdx.x;  // ((tile * hq) + h) * 4 + w
  const int w = (int)(blk & 3);
  const int32_t h = (int32_t)((blk >> 2) % hq);
  const int64_t t = (blk >> 2) / hq;
  const int tid = threadIdx.x;
  const int64_t row0 = t * kTile + 32 * w;
  if (tid < 32) {
    const int64_t row = row0 + tid;
    int live = 0, fresh = 0;
    float wr = 0.f, ws = 0.f, lv = 1.f, lnew = 0.f;
    if (row < rows) {
      const int64_t li = (int64_t)h * rows + row;
      const float l = l_s[li];
      const float lr = lse_run[li];
      if (l > 0.f) {
        const float ls = (m_s[li] + log2f(l)) * kLn2;  // the step's LSE (m in base-2 units)
        merge_weights(lr, ls, wr, ws, lnew);
        fresh = lr == kNegInf;
        lv = l;
        live = 1;
      } else {
        live = 2;  // reached by no key of this step: O_run unchanged
      }
    }
    sw_r[tid] = wr;
    sw_s[tid] = ws;
    s_l[tid] = lv;
    s_lnew[tid] = lnew;
    s_live[tid] = live;
    s_fresh[tid] = fresh;
  }
  __syncthreads();
  const float* ab = acc_s + (t * hq + h) * (int64_t)(kTile * kHeadDim) + w * (32 * kHeadDim);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int q = k * 256 + tid;                  // float4 q of the block: (4 db + i) * 64 + l + 32 hi
    const int l = q & 31, hi = (q >> 5) & 1, dbi = q >> 6;
    const int live = s_live[l];
    if (live == 0) continue;                      // row past the shard's end
    const int64_t row = row0 + l;
    const int d0 = 32 * (dbi >> 2) + 8 * (dbi & 3) + 4 * hi;
    float4* orp = (float4*)(o_run + (row * hq + h) * kHeadDim + d0);
    float4 o = *orp;
    if (live == 1) {
      const float4 a = *(const float4*)(ab + 4 * q);
      const float wr = sw_r[l], ws = sw_s[l], lv = s_l[l];
      const bool fresh = s_fresh[l] != 0;
      o = make_float4((fresh ? 0.f : wr * o.x) + ws * (a.x / lv), (fresh ? 0.f : wr * o.y) + ws * (a.y / lv),
                      (fresh ? 0.f : wr * o.z) + ws * (a.z / lv), (fresh ? 0.f : wr * o.w) + ws * (a.w / lv));
      *orp = o;
    }
    if (o_bf16) {
      __bf16 b4[4] = {(__bf16)o.x, (__bf16)o.y, (__bf16)o.z, (__bf16)o.w};
      *(uint2*)(o_bf16 + (row * hq + h) * kHeadDim + d0) = __builtin_bit_cast(uint2, b4);
    }
  }
  __syncthreads();  // every read of lse_run came before this (tid < 32 above)
  if (tid < 32 && s_live[tid] == 1) lse_run[(int64_t)h * rows + row0 + tid] = s_lnew[tid];
}

__global__ __launch_bounds__(256) void state_unpack_kernel(int64_t quads, int32_t hq, const float* o_acc,
                                                           float* out) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= quads) return;
  const int64_t e = g * 4;
  const int64_t row = e / ((int64_t)hq * kHeadDim);
  const int32_t h = (int32_t)((e / kHeadDim) % hq), d = (int32_t)(e % kHeadDim);
  *(float4*)(out + e) = *(const float4*)(o_acc + state_index(row, h, d, hq));
}

// delta[h][row] = sum_c dO[row][h][c] O[row][h][c].  One workgroup per 64 rows
// of one head: 16 lanes cover a row's 128 channels (8 each), every thread
// issues its 4 rows' loads before reducing any (8 loads of 16 bytes in
// flight), and the 64 results of the head are written as one contiguous run.
__global__ __launch_bounds__(256) void bwd_prep_kernel(int64_t rows, int32_t hq, const unsigned short* o,
                                                       const unsigned short* dout, float* delta) {
  constexpr int kRows = 64, kPass = 4;
  const int32_t h = (int32_t)(blockIdx.x % hq);
  const int64_t r0 = (int64_t)(blockIdx.x / hq) * kRows;
  const int tid = threadIdx.x, sub = tid >> 4, c8 = (tid & 15) * 8;
  uint4 a4[kPass], b4[kPass];
#pragma unroll
  for (int p = 0; p < kPass; ++p) {
    const int64_t row = r0 + p * 16 + sub;
    a4[p] = make_uint4(0, 0, 0, 0);
    b4[p] = make_uint4(0, 0, 0, 0);
    if (row < rows) {
      const int64_t off = (row * hq + h) * kHeadDim + c8;
      a4[p] = *(const uint4*)(o + off);
      b4[p] = *(const uint4*)(dout + off);
    }
  }
#pragma unroll
  for (int p = 0; p < kPass; ++p) {
    const bf16x8 av = as_bf16x8(a4[p]), bv = as_bf16x8(b4[p]);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += (float)av[i] * (float)bv[i];
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    const int64_t row = r0 + p * 16 + sub;
    if ((tid & 15) == 0 && row < rows) delta[(int64_t)h * rows + row] = s;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.nitems * a.hq;
  if (blocks <= 0) return hipSuccess;
  if (a.dense)
    hipLaunchKernelGGL(fwd_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge_bf16(int64_t rows, int32_t hq, uint16_t* o_run, float* lse_run, const uint16_t* o_s,
                             const float* lse_s, hipStream_t stream) {
  const int64_t pairs = rows * hq;
  const int64_t blocks = (pairs * 16 + 255) / 256;
  hipLaunchKernelGGL(merge_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pairs, rows, hq,
                     (unsigned short*)o_run, lse_run, (const unsigned short*)o_s, lse_s);
  return hipGetLastError();
}

hipError_t launch_merge_fp32(int64_t rows, int32_t hq, float* o_run, float* lse_run, const float* acc_s,
                             const float* m_s, const float* l_s, uint16_t* o_bf16, hipStream_t stream) {
  const int64_t tiles = (rows + kTile - 1) / kTile;
  const int64_t blocks = tiles * hq * 4;  // 32-row blocks of every (tile, head)
  hipLaunchKernelGGL(merge_fp32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, rows, hq, o_run, lse_run,
                     acc_s, m_s, l_s, (unsigned short*)o_bf16);
  return hipGetLastError();
}

hipError_t launch_state_unpack(int64_t rows, int32_t hq, const float* o_acc, float* out, hipStream_t stream) {
  const int64_t quads = rows * hq * (kHeadDim / 4);
  const int64_t blocks = (quads + 255) / 256;
  hipLaunchKernelGGL(state_unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, quads, hq, o_acc, out);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(int64_t rows, int32_t hq, const uint16_t* o,
                           const uint16_t* dout, float* delta, hipStream_t stream) {
  const int64_t blocks = (rows + 63) / 64 * hq;  // (64-row block, head)
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, rows, hq,
                     (const unsigned short*)o, (const unsigned short*)dout, delta);
  return hipGetLastError();
}

}  // namespace bsm
