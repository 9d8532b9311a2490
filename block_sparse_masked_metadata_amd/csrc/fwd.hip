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

#include "kernels.hpp"

namespace bsm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int KLD = 136;  // K tile row stride in LDS, bf16 elements (272 B)
constexpr int VLD = 160;  // V tile row stride in LDS, bf16 elements (320 B)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Two LDS transpose reads -> one 8-element MFMA operand.
__device__ inline bf16x8 lds_tr8(const unsigned short* p0, const unsigned short* p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

__device__ inline bool legal(const int4 q, const int4 k, int32_t window) {
  // tracks: x = sample, y = seg, z = noise, w = pos (MARBLE section 01)
  const int32_t d = q.w - k.w;
  const bool causal = (d >= 0) & (d < window);
  const bool span = (q.y == k.y) & (k.y >= 0);
  const bool keep = (k.z < 0) | (q.z == k.z);
  return (causal | span) & keep & (q.x == k.x);
}

__device__ inline void map_block(int32_t b, int32_t nitems, int32_t hq, int32_t hpx,
                                 int32_t& item, int32_t& h) {
  if (hpx > 0) {
    // blocks are dispatched round-robin over the 8 XCDs: give XCD x the heads
    // [x*hpx, (x+1)*hpx) so the key/value tiles of a head stay in one L2, and
    // walk its items in list order (longest first) with its heads inner.
    const int32_t x = b & 7, i = b >> 3;
    item = i / hpx;
    h = x * hpx + i % hpx;
  } else {
    item = b / hq;
    h = b % hq;
  }
  if (item >= nitems) item = -1;
}

__global__ __launch_bounds__(256, 2) void fwd_kernel(const FwdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short sK[kTile * KLD];
  __shared__ __attribute__((aligned(16))) unsigned short sV[kTile * VLD];
  __shared__ int4 sKT[kTile];

  int32_t item, h;
  map_block((int32_t)blockIdx.x, a.nitems, a.hq, a.heads_per_xcd, item, h);
  if (item < 0) return;
  const int4 it = a.items[item];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t q0 = (int64_t)it.x * kTile;
  const int64_t qi = wave * 32 + l32;
  const bool qvalid = q0 + qi < a.rows;
  const int64_t qrow = q0 + qi;
  const int32_t kvh = h / (a.hq / a.hkv);

  // Q^T as the B operand: lane holds query l32, channels [16kk + 8hi, +8).
  bf16x8 qf[8];
  {
    const unsigned short* qp = (const unsigned short*)a.q + (qrow * a.hq + h) * kHeadDim + hi * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = qvalid ? as_bf16x8(*(const uint4*)(qp + kk * 16)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  const int4 qt = qvalid ? a.qtracks[qrow] : make_int4(0, -1, -1, 0);

  // Running state.  acc[db][r] = O^T[d = 32db + 8(r/4) + 4hi + r%4][query l32].
  f32x16 acc[4];
  float mrun = kNegInf, lrun = 0.f;
  const int64_t sidx = (int64_t)h * a.rows + qrow;
  float* op = a.oacc + (qrow * a.hq + h) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  if (!(it.y & kFirst) && qvalid) {
    mrun = a.m[sidx];
    lrun = a.l[sidx];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v4 = *(const float4*)(op + db * 32 + i * 8 + hi * 4);
        acc[db][4 * i + 0] = v4.x;
        acc[db][4 * i + 1] = v4.y;
        acc[db][4 * i + 2] = v4.z;
        acc[db][4 * i + 3] = v4.w;
      }
  }

  const int64_t kstride = (int64_t)a.hkv * kHeadDim;  // elements between key rows
  const unsigned short* kbase = (const unsigned short*)a.k + (int64_t)kvh * kHeadDim;
  const unsigned short* vbase = (const unsigned short*)a.v + (int64_t)kvh * kHeadDim;

  // lane constants of the transpose reads (see the header comment)
  const int G = lane >> 4, jl = lane & 15;
  const int tr_row0 = 4 * (G >> 1) + (jl >> 2);
  const int tr_col = 16 * (G & 1) + 4 * (jl & 3);

  for (int e = 0; e < it.w; ++e) {
    const int2 ent = a.entries[it.z + e];
    const int64_t k0 = ent.x;
    const int klen = ent.y & 0xffff;
    const bool partial = (ent.y & kPartialBit) != 0;

    __syncthreads();  // previous tile's LDS readers are done
    {
      uint4 kv[8], vv[8];
      const int ch = tid & 15;
#pragma unroll
      for (int rd = 0; rd < 8; ++rd) {
        const int row = rd * 16 + (tid >> 4);
        kv[rd] = make_uint4(0, 0, 0, 0);
        vv[rd] = make_uint4(0, 0, 0, 0);
        if (row < klen) {
          kv[rd] = *(const uint4*)(kbase + (k0 + row) * kstride + ch * 8);
          vv[rd] = *(const uint4*)(vbase + (k0 + row) * kstride + ch * 8);
        }
      }
#pragma unroll
      for (int rd = 0; rd < 8; ++rd) {
        const int row = rd * 16 + (tid >> 4);
        *(uint4*)(sK + row * KLD + ch * 8) = kv[rd];
        *(uint4*)(sV + row * VLD + ch * 8) = vv[rd];
      }
      if (partial && tid < kTile)
        sKT[tid] = tid < klen ? a.ktracks[k0 + tid] : make_int4(-1, -1, -1, 0);
    }
    __syncthreads();

    // S^T = K Q^T: s[kb][r] = S[query l32][key 32kb + 8(r/4) + 4hi + r%4]
    f32x16 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const unsigned short* kr = sK + (kb * 32 + l32) * KLD + hi * 8;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 kf = as_bf16x8(*(const uint4*)(kr + kk * 16));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[kb], 0, 0, 0);
      }
    }

    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r] * a.scale_log2;
        if (partial) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (!(key < klen && legal(qt, sKT[key], a.window))) x = kNegInf;
        }
        s[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrun, mx);
    const float base = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(mrun - base);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kb][r] - base);
        s[kb][r] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32);
    lrun = lrun * alpha + ls;
    mrun = mnew;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

    // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int kb = t >> 1, hf = t & 1;
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (__bf16)s[kb][8 * hf + i];
      const unsigned short* v0 = sV + (kb * 32 + 16 * hf + tr_row0) * VLD + tr_col;
      const unsigned short* v1 = v0 + 8 * VLD;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf = lds_tr8(v0 + db * 32, v1 + db * 32);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, acc[db], 0, 0, 0);
      }
    }
  }

  if (!qvalid) return;
  if (!(it.y & kLast) || a.keep_state) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(float4*)(op + db * 32 + i * 8 + hi * 4) =
            make_float4(acc[db][4 * i], acc[db][4 * i + 1], acc[db][4 * i + 2], acc[db][4 * i + 3]);
    if (hi == 0) {
      a.m[sidx] = mrun;
      a.l[sidx] = lrun;
    }
  } else {
    // O = O_acc / l (IEEE division), then round to nearest even bf16
    const bool any = lrun > 0.f;
    unsigned short* out = (unsigned short*)a.o + (qrow * a.hq + h) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __bf16 b4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) b4[c] = (__bf16)(any ? acc[db][4 * i + c] / lrun : 0.f);
        *(uint2*)(out + db * 32 + i * 8 + hi * 4) = __builtin_bit_cast(uint2, b4);
      }
    if (hi == 0) a.lse[sidx] = lrun > 0.f ? (mrun + __log2f(lrun)) * kLn2 : kNegInf;
  }
}

__global__ __launch_bounds__(256) void bwd_prep_kernel(int64_t pairs, int64_t rows, int32_t hq,
                                                       const unsigned short* o,
                                                       const unsigned short* dout, float* delta) {
  // one thread per 8 channels; 16 lanes cover one (row, head) of 128 channels
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = gid >> 4;
  float s = 0.f;
  if (pair < pairs) {
    const uint4 a4 = *(const uint4*)(o + gid * 8);
    const uint4 b4 = *(const uint4*)(dout + gid * 8);
    const bf16x8 av = as_bf16x8(a4), bv = as_bf16x8(b4);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += (float)av[i] * (float)bv[i];
  }
  s += __shfl_xor(s, 8);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 1);
  if (pair < pairs && (gid & 15) == 0) {
    const int64_t row = pair / hq;
    const int32_t h = (int32_t)(pair % hq);
    delta[(int64_t)h * rows + row] = s;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.nitems * a.hq;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(int64_t rows, int32_t hq, const uint16_t* o,
                           const uint16_t* dout, float* delta, hipStream_t stream) {
  const int64_t pairs = rows * hq;
  const int64_t threads = pairs * 16;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pairs, rows, hq,
                     (const unsigned short*)o, (const unsigned short*)dout, delta);
  return hipGetLastError();
}

}  // namespace bsm
