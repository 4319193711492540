// Attention item of the DP: every live budget row of a sequence is a query of the new token
// at position ctx; all of them read the same cached keys/values of that sequence, so the
// cache is streamed once per (KV head, query block, context split) and staged in LDS for all
// query rows of the block (grouped-query: the hq/hkv query heads of a KV head are rows too).
//
//   qkv_finalize : sum GEMM K-splits, rotate q and k at position ctx (rotate-half RoPE with a
//                  host-computed float64 angle table), write q / own k / own v.
//   attn (MFMA)  : bf16, dh = 128.  S^T = K Q^T and O^T += V^T P^T on
//                  v_mfma_f32_32x32x16_bf16 so that each lane owns one query row's scores
//                  (softmax statistics need one cross-half exchange per 64-key tile).
//   attn (VALU)  : float32 (or any dh <= 128) reference-grade kernel, one query per lane.
//   combine      : merges the context splits (log-sum-exp) with the row's own position.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ks {

namespace {

// ------------------------------------------------------------------------------------
// q/k/v finalisation: one wave per (row, head), lane j owns the RoPE pair (j, j + dh/2).
// ------------------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void qkv_kernel(QkvArgs a) {
  const int heads = a.hq + 2 * a.hkv;
  const int widx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (widx >= a.R * heads) return;
  const int lane = threadIdx.x & 63;
  const int r = widx / heads, hd = widx % heads;
  const int half = a.dh / 2;
  const float* rope = a.rope + (size_t)a.row_seq[r] * a.dh;
  for (int j = lane; j < half; j += 64) {
    const size_t base = (size_t)r * a.ldp + (size_t)hd * a.dh;
    float x0 = a.P[base + j];
    float x1 = a.P[base + j + half];
    for (int s = 1; s < a.splits; ++s) {
      x0 += a.P[(size_t)s * a.R * a.ldp + base + j];
      x1 += a.P[(size_t)s * a.R * a.ldp + base + j + half];
    }
    if (hd < a.hq + a.hkv) {  // q and k are rotated, v is not
      const float c = rope[j], sn = rope[half + j];
      const float y0 = x0 * c - x1 * sn;
      const float y1 = x1 * c + x0 * sn;
      x0 = y0;
      x1 = y1;
    }
    if (hd < a.hq) {
      T* q = (T*)a.Q + ((size_t)r * a.hq + hd) * a.dh;
      q[j] = from_f32<T>(x0);
      q[j + half] = from_f32<T>(x1);
    } else if (hd < a.hq + a.hkv) {
      float* k = a.kself + ((size_t)r * a.hkv + (hd - a.hq)) * a.dh;
      k[j] = x0;
      k[j + half] = x1;
    } else {
      float* v = a.vself + ((size_t)r * a.hkv + (hd - a.hq - a.hkv)) * a.dh;
      v[j] = x0;
      v[j + half] = x1;
    }
  }
}

// ------------------------------------------------------------------------------------
// VALU attention partial: 64 query rows per workgroup (one per lane), keys in LDS tiles.
// ------------------------------------------------------------------------------------
constexpr int VTILE = 32;

template <class T, int DH>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a) {
  const int4 wk = a.work[blockIdx.x];
  const AttnSeq S = a.seqs[wk.x];
  const int c = wk.y, qb = wk.z, sp = wk.w;
  const int G = a.hq / a.hkv;
  const int nq = G * S.M;
  const int lane = threadIdx.x;
  const int t = qb * 64 + lane;
  const bool tvalid = t < nq;
  const int tt = tvalid ? t : nq - 1;
  const int row = S.row_off + tt / G;
  const int h = c * G + tt % G;
  const int k0 = sp * S.chunk;
  const int k1 = min(S.ctx, k0 + S.chunk);

  float q[DH], acc[DH];
  const T* qp = (const T*)a.Q + ((size_t)row * a.hq + h) * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    q[e] = to_f32(qp[e]) * a.scale_log2;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  __shared__ float Ks[VTILE][DH + 1];
  __shared__ float Vs[VTILE][DH + 1];
  const T* kb = (const T*)S.k + (size_t)c * S.cap * DH;
  const T* vb = (const T*)S.v + (size_t)c * S.cap * DH;
  for (int kt = k0; kt < k1; kt += VTILE) {
    const int nk = min(VTILE, k1 - kt);
    for (int e = lane; e < VTILE * DH; e += 64) {
      const int j = e / DH, x = e % DH;
      Ks[j][x] = j < nk ? to_f32(kb[(size_t)(kt + j) * DH + x]) : 0.f;
      Vs[j][x] = j < nk ? to_f32(vb[(size_t)(kt + j) * DH + x]) : 0.f;
    }
    __syncthreads();
    float s[VTILE];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < VTILE; ++j) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < DH; ++e) d = fmaf(q[e], Ks[j][e], d);
      s[j] = j < nk ? d : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float mn = fmaxf(m, mt);
    const float corr = exp2f(m - mn);
    l *= corr;
#pragma unroll
    for (int e = 0; e < DH; ++e) acc[e] *= corr;
#pragma unroll
    for (int j = 0; j < VTILE; ++j) {
      const float p = exp2f(s[j] - mn);
      l += p;
#pragma unroll
      for (int e = 0; e < DH; ++e) acc[e] = fmaf(p, Vs[j][e], acc[e]);
    }
    m = mn;
    __syncthreads();
  }
  if (!tvalid) return;
  const size_t qrow = (size_t)row * a.hq + h;
  const size_t slot = (size_t)sp * a.Rtot * a.hq + qrow;
  float* o = a.Opart + slot * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) o[e] = acc[e];
  a.Mpart[slot] = m;
  a.Lpart[slot] = l;
}

// ------------------------------------------------------------------------------------
// MFMA attention partial (bf16, dh = 128): 8 waves x 32 query rows = 256 query rows per
// workgroup (one workgroup per CU), 64-key tiles in a 3-stage LDS ring, so two tiles are in
// flight while one is computed.
//   * K and V tiles go global -> LDS with global_load_lds_dwordx4 (1 KB = 4 keys x 256 B per
//     wave instruction), both kept as [key][dh]; the barrier between tiles is a bare s_barrier
//     after a per-wave vmcnt wait (a fenced barrier would drain the tiles in flight).
//   * LDS has 64 banks x 4 B.  K: 16-byte chunk c of key k lives in slot c ^ (k & 15), so the
//     16-byte reads of 16 consecutive keys are conflict-free.  V: chunk c of key k lives in
//     slot c ^ (4 * (k & 3)), so the transposing reads below are conflict-free.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query's 32 scores per tile.
//   * O^T += V^T P^T: the V^T operand is read with ds_read_b64_tr_b16, which hands lane i of
//     each 16-lane group element (i % 4) of the 8 bytes addressed by lane 4e + i/4 as its
//     element e; lane (g, e, q) therefore addresses V[key 4*(g/2) + e][dh 16*(g%2) + 4q ..+3]
//     of the MFMA step and receives V^T[dh][4 consecutive keys] exactly as the MFMA wants.
//   * softmax in the log2 domain on the hardware v_exp_f32: p = 2^(s*c - m*c),
//     c = log2(e)/sqrt(dh), with a lazily raised reference m (raised, and O and l rescaled,
//     only when a score exceeds it by more than 2^8 in p); exact because l carries the same m.
// ------------------------------------------------------------------------------------
constexpr int DHM = 128;
constexpr int KT = 64;              // keys per tile
constexpr int QB = 256;             // query rows per workgroup
constexpr int NST = 3;              // LDS ring stages
constexpr float RESCALE_LOG2 = 8.f; // allowed growth of p above 1 before rescaling

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) unsigned char*)(p));
}

// s_waitcnt with vmcnt = n (n <= 15) and no wait on the other counters (gfx9 encoding)
__device__ __forceinline__ void attn_wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); break;
    case 4: __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8)); break;
    case 8: __builtin_amdgcn_s_waitcnt(8 | (7 << 4) | (15 << 8)); break;
    default: __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); break;
  }
}

__global__ __launch_bounds__(512) void attn_mfma_kernel(AttnArgs a) {
  const int4 wk = a.work[blockIdx.x];
  const AttnSeq S = a.seqs[wk.x];
  const int c = wk.y, qb = wk.z, sp = wk.w;
  const int G = a.hq / a.hkv;
  const int nq = G * S.M;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int t = qb * QB + wave * 32 + l32;
  const bool tvalid = t < nq;
  const int tt = tvalid ? t : nq - 1;
  const int row = S.row_off + tt / G;
  const int h = c * G + tt % G;
  const int k0 = sp * S.chunk;
  const int k1 = min(S.ctx, k0 + S.chunk);
  const int ntiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;
  const float cs = a.scale_log2;

  // this lane's query row as the B operand of S^T = K Q^T: 8 K-steps of 16 dh
  const bf16* qp = (const bf16*)a.Q + ((size_t)row * a.hq + h) * DHM + hi * 8;
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);

  __shared__ __attribute__((aligned(1024))) unsigned char ring[NST][2][KT * 256];

  // DMA: per stage 32 chunks (16 of K, 16 of V) of 4 keys; wave w issues chunks w + 8j.
  // Lane -> key 4*(chunk%16) + lane/16, LDS slot lane%16 <- global 16-byte chunk
  // slot ^ swz(key), swz = key & 15 for K and 4*(key & 3) for V.
  const bf16* dsrc[4];
  int dkey[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = wave + 8 * j;  // 0..31
    const int kk = 4 * (q & 15) + (lane >> 4);
    const bool isv = q >= 16;
    const int swz = isv ? 4 * (kk & 3) : (kk & 15);
    const bf16* base = (const bf16*)(isv ? S.v : S.k) + (size_t)c * S.cap * DHM;
    dsrc[j] = base + 8 * ((lane & 15) ^ swz);
    dkey[j] = kk;
  }
  auto issue = [&](int tile, int slot) {
    const int kt = k0 + tile * KT;
    const bool full = kt + KT <= k1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = wave + 8 * j;
      const int key = full ? kt + dkey[j] : min(kt + dkey[j], k1 - 1);  // clamped rows masked
      __builtin_amdgcn_global_load_lds((const void*)(dsrc[j] + (size_t)key * DHM),
                                       (void*)(&ring[slot][q >> 4][(q & 15) * 1024]), 16, 0, 0);
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY, lsum = 0.f;  // m: reference max of raw scores, shared by lanes l, l^32
  const float thresh = RESCALE_LOG2 / cs;

  // Loop-invariant LDS byte offsets within a stage.  K read for K-step ks of key l32 (+32 per
  // key block): chunk 2ks + hi in slot chunk ^ (key & 15).  V^T read (transposing) of lane
  // (g = lane/16, e = (lane/4)%4, q = lane%4) for dh block db: key 4*(g/2) + e (+ the key
  // offset of the MFMA step, a multiple of 8), dh 32db + 16(g%2) + 4q, i.e. chunk
  // 4db + 2(g%2) + q/2, half q%2, slot chunk ^ 4*(key & 3) = chunk ^ 4e.
  int koff[8], voff[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = l32 * 256 + 16 * ((2 * ks + hi) ^ (l32 & 15));
  {
    const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
    const int key = 4 * (tg >> 1) + te;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int ch = 4 * db + 2 * (tg & 1) + (tq >> 1);
      voff[db] = key * 256 + 16 * (ch ^ (4 * te)) + 8 * (tq & 1);
    }
  }
  bf16x2 ones2;
  ones2[0] = (bf16)1.f;
  ones2[1] = (bf16)1.f;

#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < ntiles) issue(p, p);

  for (int it = 0; it < ntiles; ++it) {
    attn_wait_vmcnt(4 * min(NST - 2, ntiles - 1 - it));  // this wave's part of tile `it`
    asm volatile("s_barrier" ::: "memory");              // ... and everybody else's
    if (it + NST - 1 < ntiles) issue(it + NST - 1, (it + NST - 1) % NST);
    const int kt = k0 + it * KT;
    const unsigned char* stage = &ring[it % NST][0][0];

    // scores: two 32-key blocks; lane holds query l32, keys 8*(r/4) + 4*hi + r%4
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const unsigned char* kp = stage + koff[ks];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(kp + kb * 32 * 256);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kb], 0, 0, 0);
      }
    }
    if (kt + KT > k1) {  // ragged last tile (uniform branch)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= k1) sacc[kb][r] = -INFINITY;
        }
    }
    float mt = sacc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[1][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (__builtin_amdgcn_ballot_w64(mt > m + thresh) != 0) {  // some reference too low: raise
      const float mn = mt > m + thresh ? mt : m;
      const float corr = __builtin_amdgcn_exp2f((m - mn) * cs);
      lsum *= corr;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= corr;
      m = mn;
    }
    const float mc = m * cs;

    const unsigned char* vp[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) vp[db] = stage + KT * 256 + voff[db];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[e] = (bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * st + e], cs, -mc));
        // the denominator sums exactly the rounded p that enter the P.V product
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          bf16x2 pp;
          pp[0] = pf[e];
          pp[1] = pf[e + 1];
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, lsum, false);
        }
        // V^T operand rows dh = 32db + l32, keys kb*32 + 16st + 4hi + (0..3, 8..11)
        const int kofs = (kb * 32 + 16 * st) * 256;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const s16x4 lo = lds_read_tr16(vp[db] + kofs);
          const s16x4 hv = lds_read_tr16(vp[db] + kofs + 8 * 256);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hv, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
        }
      }
    }
  }
  lsum += __shfl_xor(lsum, 32, 64);
  if (!tvalid) return;
  const size_t qrow = (size_t)row * a.hq + h;
  const size_t slot = (size_t)sp * a.Rtot * a.hq + qrow;
  float* op = a.Opart + slot * DHM;
  // O^T accumulator: lane holds dh = 32*db + 8*(r/4) + 4*hi + r%4 of query l32
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v;
      v[0] = o[db][4 * r4 + 0];
      v[1] = o[db][4 * r4 + 1];
      v[2] = o[db][4 * r4 + 2];
      v[3] = o[db][4 * r4 + 3];
      *(f32x4*)(op + 32 * db + 8 * r4 + 4 * hi) = v;
    }
  }
  if (hi == 0) {
    a.Mpart[slot] = m * cs;  // log2 domain, like the combine kernel expects
    a.Lpart[slot] = lsum;
  }
}

// ------------------------------------------------------------------------------------
// combine: one wave per (row, query head).  All maxima are in the log2 domain.
// ------------------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int widx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (widx >= a.R * a.hq) return;
  const int lane = threadIdx.x & 63;
  const int r = widx / a.hq, h = widx % a.hq;
  const int G = a.hq / a.hkv;
  const int c = h / G;
  const AttnSeq S = a.seqs[a.row_seq[r]];
  const T* q = (const T*)a.Q + ((size_t)r * a.hq + h) * a.dh;
  const float* ks = a.kself + ((size_t)r * a.hkv + c) * a.dh;
  const float* vs = a.vself + ((size_t)r * a.hkv + c) * a.dh;
  float d = 0.f;
  for (int e = lane; e < a.dh; e += 64) d = fmaf(to_f32(q[e]), ks[e], d);
  const float s_self = warp_sum(d) * a.scale_log2;
  const size_t qrow = (size_t)r * a.hq + h;
  const size_t split_stride = (size_t)a.R * a.hq;
  // lane sp < nsplit holds split sp's (max, denominator); weights 2^(m_sp - M)
  const bool has = lane < S.nsplit;
  const float ms = has ? a.Mpart[lane * split_stride + qrow] : -INFINITY;
  const float ls = has ? a.Lpart[lane * split_stride + qrow] : 0.f;
  const float mx = fmaxf(warp_max(ms), s_self);
  const float wsp = has ? exp2f(ms - mx) : 0.f;
  const float w_self = exp2f(s_self - mx);
  const float den = warp_sum(wsp * ls) + w_self;
  const float inv = 1.0f / den;
  T* out = (T*)a.O + qrow * a.dh;
  for (int e = lane; e < a.dh; e += 64) {
    float num = w_self * vs[e];
    for (int sp = 0; sp < S.nsplit; ++sp) {
      const float w = __shfl(wsp, sp, 64);
      num = fmaf(w, a.Opart[(sp * split_stride + qrow) * a.dh + e], num);
    }
    out[e] = from_f32<T>(num * inv);
  }
}

}  // namespace

int attention_qblock(int act, int dh) { return (act == ACT_BF16 && dh == 128) ? QB : 64; }
int attention_target_wgs(int act, int dh) { return (act == ACT_BF16 && dh == 128) ? 256 : 1024; }

hipError_t launch_qkv(const QkvArgs& a, int act, hipStream_t s) {
  const int waves = a.R * (a.hq + 2 * a.hkv);
  const dim3 grid((waves + 3) / 4), block(256);
  if (act == ACT_F32)
    hipLaunchKernelGGL(qkv_kernel<float>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(qkv_kernel<bf16>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int act, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  if (act == ACT_BF16 && a.dh == 128) {
    hipLaunchKernelGGL(attn_mfma_kernel, dim3(n_work), dim3(512), 0, s, a);
  } else if (act == ACT_BF16) {
    if (a.dh != 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_valu_kernel<bf16, 64>), dim3(n_work), dim3(64), 0, s, a);
  } else {
    if (a.dh == 64)
      hipLaunchKernelGGL((attn_valu_kernel<float, 64>), dim3(n_work), dim3(64), 0, s, a);
    else if (a.dh == 128)
      hipLaunchKernelGGL((attn_valu_kernel<float, 128>), dim3(n_work), dim3(64), 0, s, a);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int act, hipStream_t s) {
  const int waves = a.R * a.hq;
  const dim3 grid((waves + 3) / 4), block(256);
  if (act == ACT_F32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<bf16>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ks
