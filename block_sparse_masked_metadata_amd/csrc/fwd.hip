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
// wave w owns query rows [32w, 32w+32) of the tile.  Listed key tiles are
// processed as 64-key sub-tiles n = 0, 1, ...:
//   - S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K from LDS is the A operand,
//     Q (kept in registers for the whole item) the B operand, so the result
//     puts one query per lane (lane l and l^32 share query l%32, each holding
//     half of the sub-tile's keys) and the softmax is lane-local but for one
//     cross-lane exchange for the row max and one for the row sum, in base-2
//     units with scale*log2(e) folded into one multiply;
//   - O^T += V^T P^T on MFMA: P (bf16) is the B operand straight from the
//     registers of the softmax, with the 16 key slots of each MFMA permuted to
//     match the accumulator layout; V^T is read from the row-major V tile with
//     the gfx950 LDS transpose read (ds_read_b64_tr_b16) at the same
//     permutation.  The output accumulator again holds one query per lane, so
//     a rescale is a per-lane scalar.
// Software pipeline: iteration n runs the exponentials of S(n) beside the
// MFMAs of S(n+1), then the MFMAs of P(n) V(n) beside the row sum of P(n) and
// the mask and row max of S(n+1); a row's reference moves (rescaling O_acc and
// l) only when its max grows past it by more than 2^8, so no exponential is
// ever taken twice.  K and V reach LDS by direct-to-LDS buffer loads (no
// register staging), two buffers each: the loads of K(n+2) and V(n+1) fly
// during iteration n, with one workgroup barrier per sub-tile.

#include "tile_common.hpp"

namespace bsm {
namespace {

using dev::bf16x8;
using dev::f32x16;
using dev::kNegInf;
using dev::kLn2;
using dev::kSub;
using dev::as_bf16x8;
using dev::mfma;
using dev::lds_tr8;
using dev::legal;
using dev::query_tracks;
using dev::map_block;
using dev::in_interval;

// ---- LDS sub-tiles: 64 key rows x 256 B, unpadded, 16-byte chunks XOR-swizzled ----
// K: chunk c of row r sits in slot c ^ (r & 15), so the MFMA A-operand reads
//    (one chunk of 16 consecutive rows per 16 lanes) hit 16 distinct slots.
// V: chunk c of row r sits in slot c ^ 4(r & 3), so each transpose read
//    (4 rows x 4 chunks per 32 lanes) hits 16 distinct slots.
__device__ inline int k_slot(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
__device__ inline int v_slot(int r, int c) { return r * 256 + ((c ^ ((r & 3) << 2)) << 4); }

constexpr int kListCache = 512;           // list entries of an item kept in LDS
constexpr float kGrowth = 8.0f;           // every p stays at or below 2^8
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3: 32-bit data format, untyped loads

typedef __attribute__((address_space(3))) void lds_void;

// Sub-tile of an item: half `half` of a list entry.
struct Sub {
  int32_t k0;  // first key row
  int len;     // valid rows, 0..64
  bool partial, interval;
  int32_t ey;  // the entry word (dense-call row range and relation)
};
__device__ inline Sub sub_of(const int2 ent, int half) {
  Sub b;
  const int klen = ent.y & kLenMask;
  b.k0 = ent.x + half * kSub;
  const int len = klen - half * kSub;
  b.len = len < 0 ? 0 : (len > kSub ? kSub : len);
  b.partial = (ent.y & kPartialBit) != 0;
  b.interval = (ent.y & kIntervalBit) != 0;
  b.ey = ent.y;
  return b;
}

// Direct-to-LDS copy of one 64-row sub-tile of K or V (one KV head): wave w
// issues 4 buffer loads of 16 B per lane, load i filling rows 16i + 4w .. +3
// (1 KiB, lane l at byte 16 l).  `voff` (per lane, loop-invariant) picks each
// lane's source chunk so that the KiB holds the swizzled layout; the uniform
// row offset rides in soffset.  The record count ends at the sub-tile's last
// valid row, so rows past `len` arrive as zeros.  Byte offsets stay below
// 2^32 (a key buffer holds fewer than 2^32 bytes).
__device__ inline void dma_sub(const char* base, char* lds, const Sub& b, uint32_t row_bytes, uint32_t voff,
                               int wave) {
  // both values are uniform; readfirstlane keeps them in scalar registers (a
  // descriptor or offset held in a vector register costs a waterfall loop)
  const int nrec = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b.k0 + b.len) * row_bytes));
  const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)b.k0 * row_bytes));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nrec, kBufferFlags);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + 4096 * i + 1024 * wave), 16, voff,
                                             so + 16u * i * row_bytes, 0, 0);
}

// Mask data of key `lane` of a partial sub-tile (wave 0 stages it through a
// register): the key's tracks, its interval (lo, hi) in the first two
// fields, or with kDense its position alone.  Keys past len keep
// (-1, -1, -1, 0): sample -1 and the empty range [-1, -1) admit no query;
// with kDense they take position 2^31 - 1, outside every range.
template <bool kDense>
__device__ inline int4 key_data(const Sub& b, const int4* ktracks, const int2* kint, int lane) {
  int4 kt = make_int4(kDense ? INT32_MAX : -1, -1, -1, 0);
  if (lane < b.len) {
    if (kDense) {
      kt.x = ktracks[b.k0 + lane].w;
    } else if (b.interval) {
      const int2 iv = kint[b.k0 + lane];
      kt = make_int4(iv.x, iv.y, 0, 0);
    } else {
      kt = ktracks[b.k0 + lane];
    }
  }
  return kt;
}

// S^T = K Q^T for one staged 64-key sub-tile (unmasked):
// s[kb][r] = S[query l32][key 32kb + 8(r/4) + 4hi + r%4].
__device__ inline void qk(f32x16 (&s)[2], const char* sK, const bf16x8 (&qf)[8], int l32, int hi) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = kb * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      s[kb] = mfma(as_bf16x8(*(const uint4*)(sK + k_slot(row, 2 * kk + hi))), qf[kk], s[kb]);
  }
}

// Illegal pairs of a partial sub-tile (and keys past len) become -inf.  Every
// lane of a half-wave reads the same key's data (an LDS broadcast); no branch
// per element.  Key intervals: legal iff lo <= qc < hi (qc: the query's token
// index, -1 on pad rows), one unsigned compare.  kDense: the key position
// lies in the range dense_range gives the lane's query row `row` for the
// entry word.
template <bool kDense>
__device__ inline void mask_sub(f32x16 (&s)[2], const int4* sT, const Sub& b, const int4 qt, int32_t qc,
                                int32_t window, int hi, int row) {
  if (kDense) {
    int32_t dlo;
    uint32_t dspan;
    dense_range(b.ey, row, qt.w, window, dlo, dspan);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[kb][r] = (uint32_t)sT[key].x - (uint32_t)dlo < dspan ? s[kb][r] : kNegInf;
      }
  } else if (b.interval) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const int2 iv = *(const int2*)&sT[key];
        s[kb][r] = in_interval(qc, iv.x, iv.y) ? s[kb][r] : kNegInf;
      }
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[kb][r] = legal(qt, sT[key], window) ? s[kb][r] : kNegInf;
      }
  }
}

// The two half-waves' values of x side by side, on the vector unit (gfx950
// v_permlane32_swap trades the upper half of its first operand with the lower
// half of its second): lo holds lanes 0-31 of x in both halves, hi lanes
// 32-63, so a symmetric function of (lo, hi) is the pair's value in every
// lane, with the same operand order in both halves.  The s_nop keeps the two
// wait states the instruction needs after a vector write of its operands.
__device__ inline void half_pair(float x, float& lo, float& hi) {
  lo = x;
  hi = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}

// Row max of the sub-tile's scores in base-2 units (-inf for a row with no
// legal key): the lane's 32, then its partner half-wave's.
__device__ inline float row_max(const f32x16 (&s)[2], float c) {
  float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    m0 = fmaxf(m0, s[0][r]);
    m1 = fmaxf(m1, s[1][r]);
  }
  float lo, hi;
  half_pair(fmaxf(m0, m1), lo, hi);
  return fmaxf(lo, hi) * c;
}

// p = 2^(s c + nbase) in place, and P^T as the B operand of 4 MFMAs of 16 keys.
__device__ inline void exp_cvt(f32x16 (&s)[2], float c, float nbase, bf16x8 (&pb)[4]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, nbase));
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[t][i] = (__bf16)s[t >> 1][8 * (t & 1) + i];
}

// The row's sum of p over the sub-tile (both half-waves).
__device__ inline float row_sum(const f32x16 (&s)[2]) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    a0 += s[0][r];
    a1 += s[1][r];
  }
  float lo, hi;
  half_pair(a0 + a1, lo, hi);
  return lo + hi;
}

// Lane constants of the V transpose reads.
struct TrV {
  int row0, chunk, off8;
  __device__ inline explicit TrV(int lane) {
    const int G = lane >> 4, jl = lane & 15;
    row0 = 4 * (G >> 1) + (jl >> 2);
    chunk = 2 * (G & 1) + ((jl & 3) >> 1);  // + 4 db
    off8 = (jl & 1) * 8;
  }
};

// O^T += V^T P^T over one staged sub-tile, 16 keys per MFMA (the 8 transpose
// reads of a key group first).
__device__ inline void pv(f32x16 (&acc)[4], const char* sV, const bf16x8 (&pb)[4], const TrV& tr) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r0 = 16 * t + tr.row0;
    bf16x8 vf[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
      vf[db] = lds_tr8(sV + v_slot(r0, 4 * db + tr.chunk) + tr.off8, sV + v_slot(r0 + 8, 4 * db + tr.chunk) + tr.off8);
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = mfma(vf[db], pb[t], acc[db]);
  }
}

// Lazy reference: when some row's max mt (base 2) exceeds its reference by
// more than 2^kGrowth, every row whose max is above its reference moves the
// reference there and rescales O_acc and l by 2^(old - new) (0 from -inf).
// O_acc and l always share one reference, so the result is exact either way.
__device__ inline void move_reference(float mt, float& mref, float& lrun, f32x16 (&acc)[4], float& nbase) {
  if (__any(mt > mref + kGrowth)) {
    const float mnew = fmaxf(mref, mt);
    const float alpha = mnew == mref ? 1.f : __builtin_amdgcn_exp2f(mref - mnew);
    lrun *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    mref = mnew;
    nbase = mref == kNegInf ? 0.f : -mref;
  }
}

template <bool kDense>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char sK0[kSub * 256];
  __shared__ __attribute__((aligned(1024))) char sK1[kSub * 256];
  __shared__ __attribute__((aligned(1024))) char sV0[kSub * 256];
  __shared__ __attribute__((aligned(1024))) char sV1[kSub * 256];
  __shared__ int4 sT0[kSub];
  __shared__ int4 sT1[kSub];
  __shared__ int2 sEnt[kListCache];

  int32_t item, h;
  map_block((int32_t)blockIdx.x, a.nitems, a.hq, a.heads_per_xcd, item, h);
  if (item < 0) return;
  // Prologue in two memory round trips: the item record and its first list
  // entry (scalar loads, side by side), then every other load at once: the
  // list, K of sub-tiles 0 and 1 and V of sub-tile 0 (the two halves of the
  // first entry), their mask data, Q, the query tracks and the state.
  int4 it = a.items[item];
  if (a.step_only) it.y = kFirst | kLast;  // this step's keys alone
  int2 ent = a.first[item];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // source chunk of this lane's 16 bytes in each direct-to-LDS load: row
  // 16i + rw of the sub-tile, slot lane % 16
  const int rw = 4 * wave + (lane >> 4);
  const uint32_t koff = (uint32_t)rw * row_bytes + 16u * (uint32_t)((lane & 15) ^ (rw & 15));
  const uint32_t voff = (uint32_t)rw * row_bytes + 16u * (uint32_t)((lane & 15) ^ ((rw & 3) << 2));
  const float c = a.scale_log2;

  ent.x = __builtin_amdgcn_readfirstlane(ent.x);
  ent.y = __builtin_amdgcn_readfirstlane(ent.y);
  const Sub b0 = sub_of(ent, 0), b1 = sub_of(ent, 1);
  const bool stage0 = b0.partial && wave == 0;
  int4 t0 = make_int4(0, 0, 0, 0), t1 = make_int4(0, 0, 0, 0);
  if (stage0) {
    t0 = key_data<kDense>(b0, a.ktracks, a.kint, lane);
    t1 = key_data<kDense>(b1, a.ktracks, a.kint, lane);
  }
  dma_sub(kbase, sK0, b0, row_bytes, koff, wave);
  dma_sub(vbase, sV0, b0, row_bytes, voff, wave);
  dma_sub(kbase, sK1, b1, row_bytes, koff, wave);

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
  if (stage0) {
    sT0[lane] = t0;
    sT1[lane] = t1;
  }
  // Drain every prologue load here, once (the direct-to-LDS loads included).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const TrV tr(lane);
  float nbase = mref == kNegInf ? 0.f : -mref;
  f32x16 s0[2], s1[2];
  qk(s0, sK0, qf, l32, hi);
  if (b0.partial) mask_sub<kDense>(s0, sT0, b0, qt, qc, a.window, hi, (int)qi);
  move_reference(row_max(s0, c), mref, lrun, acc, nbase);

  // Sub-tiles in pairs (2e, 2e + 1) = the halves of entry e.  Buffers: K of
  // even sub-tiles in sK0, odd in sK1; V and mask data likewise.  At the top
  // of iteration n, S(n) is in registers (masked, reference moved), K(n+1),
  // V(n) and the mask data of n+1 are in LDS.
  int2 entE = ent;
  for (int e = 0; e < it.w; ++e) {
    const bool more = e + 1 < it.w;  // sub-tiles 2e + 2 and 2e + 3 exist
    __syncthreads();  // every wave is done with sub-tile 2e - 1's V, 2e's K and mask data
    int2 entF = entE;
    if (more) {
      const int e1 = e + 1;
      if (e1 % kListCache == 0) {  // next chunk of the list (long lists only)
        for (int i = tid; i < kListCache && e1 + i < it.w; i += 256) sEnt[i] = a.entries[it.z + e1 + i];
        __syncthreads();
      }
      entF = sEnt[e1 % kListCache];
      entF.x = __builtin_amdgcn_readfirstlane(entF.x);
      entF.y = __builtin_amdgcn_readfirstlane(entF.y);
    }
    {  // n = 2e: S(n) in s0
      const Sub bn = sub_of(entE, 1), bl = sub_of(entF, 0);  // sub-tiles n + 1, n + 2
      const bool stage = more && bl.partial && wave == 0;
      int4 tl = make_int4(0, 0, 0, 0);
      if (stage) tl = key_data<kDense>(bl, a.ktracks, a.kint, lane);
      if (more) dma_sub(kbase, sK0, bl, row_bytes, koff, wave);
      dma_sub(vbase, sV1, bn, row_bytes, voff, wave);
      bf16x8 pb[4];
      qk(s1, sK1, qf, l32, hi);
      exp_cvt(s0, c, nbase, pb);
      pv(acc, sV0, pb, tr);
      lrun += row_sum(s0);
      if (bn.partial) mask_sub<kDense>(s1, sT1, bn, qt, qc, a.window, hi, (int)qi);
      move_reference(row_max(s1, c), mref, lrun, acc, nbase);
      if (stage) sT0[lane] = tl;
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of K(n+2), V(n+1) have landed
    }
    __syncthreads();  // every wave is done with sub-tile 2e's V, 2e + 1's K and mask data
    {  // n = 2e + 1: S(n) in s1
      const Sub bn = sub_of(entF, 0), bl = sub_of(entF, 1);  // sub-tiles n + 1, n + 2 (when more)
      const bool stage = more && bl.partial && wave == 0;
      int4 tl = make_int4(0, 0, 0, 0);
      if (stage) tl = key_data<kDense>(bl, a.ktracks, a.kint, lane);
      if (more) {
        dma_sub(kbase, sK1, bl, row_bytes, koff, wave);
        dma_sub(vbase, sV0, bn, row_bytes, voff, wave);
      }
      bf16x8 pb[4];
      if (more) qk(s0, sK0, qf, l32, hi);
      exp_cvt(s1, c, nbase, pb);
      pv(acc, sV1, pb, tr);
      lrun += row_sum(s1);
      if (more) {
        if (bn.partial) mask_sub<kDense>(s0, sT0, bn, qt, qc, a.window, hi, (int)qi);
        move_reference(row_max(s0, c), mref, lrun, acc, nbase);
      }
      if (stage) sT1[lane] = tl;
      __builtin_amdgcn_s_waitcnt(0x0f70);
    }
    entE = entF;
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
        for (int cc = 0; cc < 4; ++cc) b4[cc] = (__bf16)(acc[db][4 * i + cc] * rl);
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
