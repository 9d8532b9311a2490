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
//          list; S^T and dP^T put one query per lane, so LSE_i and D_i are
//          lane scalars; dQ^T += K^T dS^T reads K^T with the LDS transpose
//          read.
//   dkdv : one workgroup per (key tile, key/value head), walking the tile's
//          column list and every query head of the group; S and dP put one
//          key per lane; dV^T += dO^T P and dK^T += Q^T dS read dO^T and Q^T
//          with the LDS transpose read.  K and V rows stay in registers.

#include "kernels.hpp"

namespace bsm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int LD = 136;  // LDS row stride of a staged 128x128 tile (bf16 elements)
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kInf = __builtin_inff();

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline bf16x8 lds_tr8(const unsigned short* p0, const unsigned short* p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

__device__ inline bool legal(const int4 q, const int4 k, int32_t window) {
  const int32_t d = q.w - k.w;
  const bool causal = (d >= 0) & (d < window);
  const bool span = (q.y == k.y) & (k.y >= 0);
  const bool keep = (k.z < 0) | (q.z == k.z);
  return (causal | span) & keep & (q.x == k.x);
}

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

// Stage rows [r0, r0+len) of a [rows, H, 128] bf16 tensor (head h) into a
// padded LDS tile; rows >= len are zero.
__device__ inline void stage_tile(unsigned short* dst, const unsigned short* src, int64_t r0,
                                  int len, int64_t row_stride, int tid) {
  uint4 v[8];
  const int ch = tid & 15;
#pragma unroll
  for (int rd = 0; rd < 8; ++rd) {
    const int row = rd * 16 + (tid >> 4);
    v[rd] = make_uint4(0, 0, 0, 0);
    if (row < len) v[rd] = *(const uint4*)(src + (r0 + row) * row_stride + ch * 8);
  }
#pragma unroll
  for (int rd = 0; rd < 8; ++rd) {
    const int row = rd * 16 + (tid >> 4);
    *(uint4*)(dst + row * LD + ch * 8) = v[rd];
  }
}

__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short sK[kTile * LD];
  __shared__ __attribute__((aligned(16))) unsigned short sV[kTile * LD];
  __shared__ int4 sKT[kTile];

  int32_t item, h;
  map_block((int32_t)blockIdx.x, a.nitems, a.hq, a.heads_per_xcd, item, h);
  if (item < 0) return;
  const int4 it = a.items[item];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t qrow = (int64_t)it.x * kTile + wave * 32 + l32;
  const bool qvalid = qrow < a.rows;
  const int32_t kvh = h / (a.hq / a.hkv);

  bf16x8 qf[8], df[8];
  {
    const int64_t off = (qrow * a.hq + h) * kHeadDim + hi * 8;
    const unsigned short* qp = (const unsigned short*)a.q + off;
    const unsigned short* dp = (const unsigned short*)a.dout + off;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = qvalid ? as_bf16x8(*(const uint4*)(qp + kk * 16)) : as_bf16x8(make_uint4(0, 0, 0, 0));
      df[kk] = qvalid ? as_bf16x8(*(const uint4*)(dp + kk * 16)) : as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  const int64_t sidx = (int64_t)h * a.rows + qrow;
  const float lse2 = qvalid ? a.lse[sidx] * kLog2e : kInf;
  const float dl = qvalid ? a.delta[sidx] : 0.f;
  const int4 qt = qvalid ? a.qtracks[qrow] : make_int4(0, -1, -1, 0);

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  const int64_t kstride = (int64_t)a.hkv * kHeadDim;
  const unsigned short* kbase = (const unsigned short*)a.k + (int64_t)kvh * kHeadDim;
  const unsigned short* vbase = (const unsigned short*)a.v + (int64_t)kvh * kHeadDim;
  const int G = lane >> 4, jl = lane & 15;
  const int tr_row0 = 4 * (G >> 1) + (jl >> 2);
  const int tr_col = 16 * (G & 1) + 4 * (jl & 3);

  for (int e = 0; e < it.w; ++e) {
    const int2 ent = a.entries[it.z + e];
    const int64_t k0 = ent.x;
    const int klen = ent.y & 0xffff;
    const bool partial = (ent.y & kPartialBit) != 0;
    __syncthreads();
    stage_tile(sK, kbase, k0, klen, kstride, tid);
    stage_tile(sV, vbase, k0, klen, kstride, tid);
    if (partial && tid < kTile) sKT[tid] = tid < klen ? a.ktracks[k0 + tid] : make_int4(-1, -1, -1, 0);
    __syncthreads();

#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int kb = 2 * half + k2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[k2][r] = 0.f;
          dp[k2][r] = 0.f;
        }
        const unsigned short* kr = sK + (kb * 32 + l32) * LD + hi * 8;
        const unsigned short* vr = sV + (kb * 32 + l32) * LD + hi * 8;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          s[k2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*(const uint4*)(kr + kk * 16)), qf[kk], s[k2], 0, 0, 0);
          dp[k2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*(const uint4*)(vr + kk * 16)), df[kk], dp[k2], 0, 0, 0);
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = (2 * half + k2) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          bool ok = true;
          if (partial) ok = key < klen && legal(qt, sKT[key], a.window);
          const float p = ok ? __builtin_amdgcn_exp2f(s[k2][r] * a.scale_log2 - lse2) : 0.f;
          dp[k2][r] = p * (dp[k2][r] - dl);
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k2 = t >> 1, hf = t & 1;
        const int kb = 2 * half + k2;
        bf16x8 dsb;
#pragma unroll
        for (int i = 0; i < 8; ++i) dsb[i] = (__bf16)dp[k2][8 * hf + i];
        const unsigned short* k0p = sK + (kb * 32 + 16 * hf + tr_row0) * LD + tr_col;
        const unsigned short* k1p = k0p + 8 * LD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr8(k0p + db * 32, k1p + db * 32), dsb, acc[db], 0, 0, 0);
      }
    }
  }

  if (!qvalid) return;
  float* out = a.dq + (qrow * a.hq + h) * kHeadDim;
  const bool first = (it.y & kFirst) != 0;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* p = out + db * 32 + i * 8 + hi * 4;
      float4 o4 = first ? make_float4(0.f, 0.f, 0.f, 0.f) : *(const float4*)p;
      o4.x += a.scale * acc[db][4 * i + 0];
      o4.y += a.scale * acc[db][4 * i + 1];
      o4.z += a.scale * acc[db][4 * i + 2];
      o4.w += a.scale * acc[db][4 * i + 3];
      *(float4*)p = o4;
    }
}

__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short sQ[kTile * LD];
  __shared__ __attribute__((aligned(16))) unsigned short sO[kTile * LD];
  __shared__ float sL[kTile];
  __shared__ float sD[kTile];
  __shared__ int4 sQT[kTile];

  int32_t item, g;
  map_block((int32_t)blockIdx.x, a.nitems, a.hkv, a.heads_per_xcd, item, g);
  if (item < 0) return;
  const int4 it = a.items[item];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int kl = wave * 32 + l32;
  const int64_t key = (int64_t)it.x * kTile + kl;
  const bool kvalid = key < a.krows;
  const int32_t grp = a.hq / a.hkv;

  bf16x8 kf[8], vf[8];
  {
    const int64_t off = (key * a.hkv + g) * kHeadDim + hi * 8;
    const unsigned short* kp = (const unsigned short*)a.k + off;
    const unsigned short* vp = (const unsigned short*)a.v + off;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      kf[kk] = kvalid ? as_bf16x8(*(const uint4*)(kp + kk * 16)) : as_bf16x8(make_uint4(0, 0, 0, 0));
      vf[kk] = kvalid ? as_bf16x8(*(const uint4*)(vp + kk * 16)) : as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  const int4 kt = kvalid ? a.ktracks[key] : make_int4(-1, -1, -1, 0);

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  const int64_t qstride = (int64_t)a.hq * kHeadDim;
  const int G = lane >> 4, jl = lane & 15;
  const int tr_row0 = 4 * (G >> 1) + (jl >> 2);
  const int tr_col = 16 * (G & 1) + 4 * (jl & 3);

  for (int hh = 0; hh < grp; ++hh) {
    const int32_t h = g * grp + hh;
    const unsigned short* qbase = (const unsigned short*)a.q + (int64_t)h * kHeadDim;
    const unsigned short* obase = (const unsigned short*)a.dout + (int64_t)h * kHeadDim;
    for (int e = 0; e < it.w; ++e) {
      const int2 ent = a.entries[it.z + e];
      const int64_t q0 = ent.x;
      const int qlen = ent.y & 0xffff;
      const bool partial = (ent.y & kPartialBit) != 0;
      __syncthreads();
      stage_tile(sQ, qbase, q0, qlen, qstride, tid);
      stage_tile(sO, obase, q0, qlen, qstride, tid);
      if (tid < kTile) {
        const bool ok = tid < qlen;
        sL[tid] = ok ? a.lse[(int64_t)h * a.rows + q0 + tid] * kLog2e : kInf;
        sD[tid] = ok ? a.delta[(int64_t)h * a.rows + q0 + tid] : 0.f;
        if (partial) sQT[tid] = ok ? a.qtracks[q0 + tid] : make_int4(-2, -1, -1, 0);
      }
      __syncthreads();

#pragma unroll
      for (int qc = 0; qc < 4; ++qc) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = 0.f;
          dp[r] = 0.f;
        }
        const unsigned short* qr = sQ + (qc * 32 + l32) * LD + hi * 8;
        const unsigned short* orow = sO + (qc * 32 + l32) * LD + hi * 8;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*(const uint4*)(qr + kk * 16)), kf[kk], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*(const uint4*)(orow + kk * 16)), vf[kk], dp, 0, 0, 0);
        }
        // lane: key kl; register r: query qc*32 + 8(r/4) + 4hi + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qc * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          bool ok = true;
          if (partial) ok = qi < qlen && legal(sQT[qi], kt, a.window);
          const float p = ok ? __builtin_amdgcn_exp2f(s[r] * a.scale_log2 - sL[qi]) : 0.f;
          s[r] = p;
          dp[r] = p * (dp[r] - sD[qi]);
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          bf16x8 pb, dsb;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            pb[i] = (__bf16)s[8 * hf + i];
            dsb[i] = (__bf16)dp[8 * hf + i];
          }
          const int row0 = (qc * 32 + 16 * hf + tr_row0) * LD + tr_col;
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x8 of = lds_tr8(sO + row0 + db * 32, sO + row0 + 8 * LD + db * 32);
            dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(of, pb, dv[db], 0, 0, 0);
            const bf16x8 qfv = lds_tr8(sQ + row0 + db * 32, sQ + row0 + 8 * LD + db * 32);
            dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfv, dsb, dk[db], 0, 0, 0);
          }
        }
      }
    }
  }

  if (!kvalid) return;
  const int64_t off = (key * a.hkv + g) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = db * 32 + i * 8 + hi * 4;
      float4 k4 = *(const float4*)(a.dk + off + c);
      float4 v4 = *(const float4*)(a.dv + off + c);
      k4.x += a.scale * dk[db][4 * i + 0];
      k4.y += a.scale * dk[db][4 * i + 1];
      k4.z += a.scale * dk[db][4 * i + 2];
      k4.w += a.scale * dk[db][4 * i + 3];
      v4.x += dv[db][4 * i + 0];
      v4.y += dv[db][4 * i + 1];
      v4.z += dv[db][4 * i + 2];
      v4.w += dv[db][4 * i + 3];
      *(float4*)(a.dk + off + c) = k4;
      *(float4*)(a.dv + off + c) = v4;
    }
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.nitems * a.hq;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.nitems * a.hkv;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsm
