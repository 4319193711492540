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
// MFMA attention partial (bf16, dh = 128): 4 waves x 32 query rows, 64-key tiles.
//   * the next tile's K/V are loaded into registers while the current tile is computed,
//     then written to the other LDS buffer: one barrier per tile;
//   * threads 0..127 stage K rows as they are ([key][dh]); threads 128..255 each load an
//     8-key x 8-dh block of V, transpose it in registers and store 8-key rows of V^T, so the
//     P.V MFMA reads its operand with 8-byte LDS loads;
//   * softmax in the log2 domain on raw scores: p = exp2(s*c - m*c), c = log2(e)/sqrt(dh);
//     the O rescale is skipped when no lane's running max moved.
// ------------------------------------------------------------------------------------
constexpr int DHM = 128;
constexpr int KT = 64;            // keys per tile
constexpr int K_PITCH = DHM + 8;  // LDS row pitch of K [key][dh] (bf16 elements)
constexpr int V_PITCH = KT + 8;   // LDS row pitch of V^T [dh][key]

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs a) {
  const int4 wk = a.work[blockIdx.x];
  const AttnSeq S = a.seqs[wk.x];
  const int c = wk.y, qb = wk.z, sp = wk.w;
  const int G = a.hq / a.hkv;
  const int nq = G * S.M;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int t = qb * 128 + wave * 32 + l32;
  const bool tvalid = t < nq;
  const int tt = tvalid ? t : nq - 1;
  const int row = S.row_off + tt / G;
  const int h = c * G + tt % G;
  const int k0 = sp * S.chunk;
  const int k1 = min(S.ctx, k0 + S.chunk);
  const float cs = a.scale_log2;

  // this lane's query row as the B operand of S^T = K Q^T: 8 K-steps of 16 dh
  const bf16* qp = (const bf16*)a.Q + ((size_t)row * a.hq + h) * DHM + hi * 8;
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);

  __shared__ bf16 Ks[2][KT * K_PITCH];
  __shared__ bf16 Vt[2][DHM * V_PITCH];

  const bf16* kbase = (const bf16*)S.k + (size_t)c * S.cap * DHM;
  const bf16* vbase = (const bf16*)S.v + (size_t)c * S.cap * DHM;
  const bool k_role = tid < 128;
  const int u = tid & 127;
  bf16x8 stg[8];
  bf16x8 zero8;
#pragma unroll
  for (int e = 0; e < 8; ++e) zero8[e] = (bf16)0.f;

  auto load_tile = [&](int kt) {
    if (k_role) {
      const int key = kt + (u >> 1);
      const bf16* src = kbase + (size_t)key * DHM + (u & 1) * 64;
#pragma unroll
      for (int e = 0; e < 8; ++e) stg[e] = key < k1 ? *(const bf16x8*)(src + 8 * e) : zero8;
    } else {
      const int kb8 = u & 7, j = u >> 3;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int key = kt + 8 * kb8 + r;
        stg[r] = key < k1 ? *(const bf16x8*)(vbase + (size_t)key * DHM + 8 * j) : zero8;
      }
    }
  };
  auto store_tile = [&](int buf) {
    if (k_role) {
      bf16* dst = &Ks[buf][(u >> 1) * K_PITCH + (u & 1) * 64];
#pragma unroll
      for (int e = 0; e < 8; ++e) *(bf16x8*)(dst + 8 * e) = stg[e];
    } else {
      // stg[r] holds V[key 8*kb8 + r][dh 8j .. 8j+7]; word k of it = dh pair (2k, 2k+1).
      // Column cc of the block (dh 8j + cc) as 8 keys: word m = (V[2m][cc], V[2m+1][cc]).
      const int kb8 = u & 7, j = u >> 3;
      u32x4 w[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) w[r] = as_u32x4(stg[r]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          u32x4 col;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const unsigned lo = w[2 * m][k], hw = w[2 * m + 1][k];
            col[m] = b == 0 ? ((lo & 0xFFFFu) | (hw << 16)) : ((lo >> 16) | (hw & 0xFFFF0000u));
          }
          *(u32x4*)(&Vt[buf][(8 * j + 2 * k + b) * V_PITCH + 8 * kb8]) = col;
        }
      }
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  int buf = 0;
  if (k0 < k1) {
    load_tile(k0);
    store_tile(0);
  }
  __syncthreads();
  for (int kt = k0; kt < k1; kt += KT) {
    const bool more = kt + KT < k1;
    if (more) load_tile(kt + KT);

    // scores: two 32-key blocks; lane holds query l32, keys 8*(r/4) + 4*hi + r%4
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf =
            *(const bf16x8*)(&Ks[buf][(kb * 32 + l32) * K_PITCH + ks * 16 + hi * 8]);
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
    const float mn = fmaxf(m, mt);
    if (__builtin_amdgcn_ballot_w64(mn > m) != 0) {  // some running max moved: rescale
      const float corr = exp2f((m - mn) * cs);
      lsum *= corr;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= corr;
    }
    m = mn;
    const float mc = mn * cs;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2f(fmaf(sacc[kb][8 * st + e], cs, -mc));
          lsum += p;
          pf[e] = (bf16)p;
        }
        // V^T operand: keys kb*32 + 16*st + 8*(e/4) + 4*hi + e%4 for e = 0..7
        const int kofs = kb * 32 + 16 * st + 4 * hi;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16* vrow = &Vt[buf][(db * 32 + l32) * V_PITCH + kofs];
          const bf16x4 lo = *(const bf16x4*)(vrow);
          const bf16x4 hv = *(const bf16x4*)(vrow + 8);
          const bf16x8 vf = __builtin_shufflevector(lo, hv, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
        }
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
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
  float mx = s_self;
  for (int sp = 0; sp < S.nsplit; ++sp) mx = fmaxf(mx, a.Mpart[sp * split_stride + qrow]);
  const float w_self = exp2f(s_self - mx);
  float den = w_self;
  for (int sp = 0; sp < S.nsplit; ++sp) {
    const float ms = a.Mpart[sp * split_stride + qrow];
    den += exp2f(ms - mx) * a.Lpart[sp * split_stride + qrow];
  }
  const float inv = 1.0f / den;
  T* out = (T*)a.O + qrow * a.dh;
  for (int e = lane; e < a.dh; e += 64) {
    float num = w_self * vs[e];
    for (int sp = 0; sp < S.nsplit; ++sp) {
      const float ms = a.Mpart[sp * split_stride + qrow];
      const float wsp = exp2f(ms - mx);
      num = fmaf(wsp, a.Opart[(sp * split_stride + qrow) * a.dh + e], num);
    }
    out[e] = from_f32<T>(num * inv);
  }
}

}  // namespace

int attention_qblock(int act, int dh) { return (act == ACT_BF16 && dh == 128) ? 128 : 64; }

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
    hipLaunchKernelGGL(attn_mfma_kernel, dim3(n_work), dim3(256), 0, s, a);
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
