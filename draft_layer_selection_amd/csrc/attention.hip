// Attention item of the DP: every live budget row of a sequence is a query of the new token
// at position ctx; all of them read the same cached keys/values of that sequence, so the
// cache is streamed once per (KV head, query block, context split) and staged in LDS for all
// query rows of the block (grouped-query: the hq/hkv query heads of a KV head are rows too).
//
//   qkv_finalize : sum GEMM K-splits, rotate q and k at position ctx (rotate-half RoPE with a
//                  host-computed float64 angle table), write q (bf16: times log2(e)/sqrt(dh),
//                  the MFMA kernel's score units) / own k / own v.
//   attn (MFMA)  : bf16, dh = 128 or 64.  S^T = K Q^T and O^T += V^T P^T on
//                  v_mfma_f32_32x32x16_bf16 so that each lane owns one query row's scores
//                  (softmax statistics need one cross-half exchange per 64-key tile).
//   attn (VALU)  : float32 (or any dh <= 128) reference-grade kernel, one query per lane.
//   combine      : merges the context splits (log-sum-exp) with the row's own position.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ks {

namespace {

// ------------------------------------------------------------------------------------
// q/k/v finalisation: one wave per (row, head), lane j owns the RoPE pair (j, j + dh/2)
// (dh <= 128, so one pair per lane).
// ------------------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void qkv_kernel(QkvArgs a) {
  const int heads = a.hq + 2 * a.hkv;
  // wave-uniform: the row's metadata come through scalar loads
  const int widx = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (widx >= a.R * heads) return;
  const int j = threadIdx.x & 63;
  const int half = a.dh / 2;
  if (j >= half) return;
  const int r = widx / heads, hd = widx % heads;
  const size_t split_stride = (size_t)a.R * a.ldp;
  const size_t base = (size_t)r * a.ldp + (size_t)hd * a.dh;
  // every split's loads in flight before the first addition; the sum keeps the split order
  float p0[GEMM_MAX_SPLITS], p1[GEMM_MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < GEMM_MAX_SPLITS; ++s)
    if (s < a.splits) {
      p0[s] = a.P[s * split_stride + base + j];
      p1[s] = a.P[s * split_stride + base + j + half];
    }
  // the row's RoPE pair, loaded for v heads too so that its loads overlap the splits'
  const float* rope = a.rope + ((size_t)a.row_seq[r] * a.wmax + a.row_tok[r]) * a.dh;
  const float c = rope[j], sn = rope[half + j];
  float x0 = p0[0], x1 = p1[0];
#pragma unroll
  for (int s = 1; s < GEMM_MAX_SPLITS; ++s)
    if (s < a.splits) {
      x0 += p0[s];
      x1 += p1[s];
    }
  if (hd < a.hq + a.hkv) {  // q and k are rotated, v is not
    const float y0 = x0 * c - x1 * sn;
    const float y1 = x1 * c + x0 * sn;
    x0 = y0;
    x1 = y1;
  }
  if (hd < a.hq) {
    T* q = (T*)a.Q + ((size_t)r * a.hq + hd) * a.dh;
    q[j] = from_f32<T>(x0 * a.q_scale);
    q[j + half] = from_f32<T>(x1 * a.q_scale);
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

// ------------------------------------------------------------------------------------
// VALU attention partial: 64 query rows per workgroup (one per lane), keys in LDS tiles.
// ------------------------------------------------------------------------------------
constexpr int VTILE = 32;

template <class T, int DH>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a) {
  const int4 wk = a.work[blockIdx.x];
  if (wk.x < 0) return;
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
  const size_t slot = attn_slot(S, sp, tt / G, a.hq, h);
  float* o = a.Opart + slot * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) o[e] = acc[e];
  a.Mpart[slot] = m;
  a.Lpart[slot] = l;
}

// ------------------------------------------------------------------------------------
// MFMA attention partial (bf16, dh = 128 or 64): 8 waves x 32 query rows = 256 query rows per
// workgroup (one workgroup per CU), 64-key tiles.  The layout notes below are for dh = 128;
// AttnGeom states the dh = 64 swizzles.
//   * K and V tiles are loaded with range-checked 16-byte buffer loads into registers one
//     iteration ahead and stored to a K ring and a V ring of four slots each, both kept as
//     [key][dh] (measured faster than loading global -> LDS directly, which competes with the
//     LDS reads of the MFMA operands).
//   * LDS has 64 banks x 4 B.  K: 16-byte chunk c of key k lives in slot c ^ (k & 15), so the
//     16-byte reads of 16 consecutive keys are conflict-free.  V: chunk c of key k lives in
//     slot c ^ (4 * (k & 3)), so the transposing reads below are conflict-free.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query's 32 scores per tile.
//   * O^T += V^T P^T: the V^T operand is read with ds_read_b64_tr_b16, which hands lane i of
//     each 16-lane group element (i % 4) of the 8 bytes addressed by lane 4e + i/4 as its
//     element e; lane (g, e, q) therefore addresses V[key 4*(g/2) + e][dh 16*(g%2) + 4q ..+3]
//     of the MFMA step and receives V^T[dh][4 consecutive keys] exactly as the MFMA wants.
//   * softmax in the log2 domain on the hardware v_exp_f32: q is stored times
//     c = log2(e)/sqrt(dh) (by the q/k/v finalisation), so a score q.k is already in the
//     exponent's units, and the first score MFMA of a tile starts from -m instead of 0: the
//     accumulators hold q.k - m and p = 2^(accumulator), with no per-score shift.  The
//     reference m is raised lazily (and O, l and the tile's scores shifted) only when a score
//     exceeds it by more than 8, i.e. p above 2^8; exact because l carries the same m.
//   * Software pipeline: iteration t issues the score MFMAs of tile t+1 between the
//     exponentials and P.V MFMAs of tile t, so one wave keeps the matrix core and the vector
//     ALU busy at once.  K of tile t is read in iteration t-1 and V in iteration t; tile t is
//     loaded in iteration t-3 and stored to LDS in iteration t-2.
// ------------------------------------------------------------------------------------
constexpr int KT = 64;                 // keys per tile
constexpr int QB = 256;                // query rows per workgroup
constexpr int NR = 4;                  // slots of the K ring and of the V ring
constexpr float RESCALE_LOG2 = 8.f;    // allowed growth of p above 1 before rescaling

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// transposing LDS read at an LDS-space byte address (kept in LDS space so the constant part
// of the address folds into the instruction's offset field)
__device__ __forceinline__ s16x4 lds_read_tr16(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// max / sum of a value over the lane pair (l, l ^ 32) with one v_permlane32_swap
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt with vmcnt = 0 only, and with lgkmcnt = 0 only (gfx9 encoding: vmcnt bits [3:0]
// and [15:14], expcnt [6:4], lgkmcnt [11:8]); the barrier between tiles is a bare s_barrier
// after these, since __syncthreads would also drain the staged loads in flight
__device__ __forceinline__ void attn_wait_vmcnt(int) {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void attn_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Head sizes 128 and 64.  A key's row of K or V is ROWB = 2*DH bytes: 16 chunks of 16 bytes at
// DH = 128, 8 at DH = 64; the swizzles below keep both the 16-byte K reads and the transposing
// V reads conflict-free (16 consecutive keys, resp. the 32 lanes of a read phase, on distinct
// 16-byte slots modulo 256 bytes).
template <int DH>
struct AttnGeom {
  static constexpr int ROWB = 2 * DH;
  static constexpr int TB = KT * ROWB;            // bytes of one K (or V) tile
  static constexpr int CPW = TB / 1024 / 8;       // 1 KB load chunks per wave per tile
  static constexpr int LPR = ROWB / 16;           // lanes per key row in a load chunk
  static constexpr int KSTEPS = DH / 16;          // 16-wide steps of q . k
  static constexpr int DB = DH / 32;              // 32-row dh blocks of O^T
  // slot of 16-byte chunk c of key k: K read by 16 consecutive keys, V by the transposing read
  static __device__ __forceinline__ int swz_k(int k) { return DH == 128 ? (k & 15) : ((k >> 1) & 7); }
  static __device__ __forceinline__ int swz_v(int k) { return DH == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); }
};

template <int DH>
__global__ __launch_bounds__(512) void attn_mfma_kernel(AttnArgs a) {
  using Geo = AttnGeom<DH>;
  constexpr int ROWB = Geo::ROWB, TILE_BYTES = Geo::TB, CPW = Geo::CPW, LPR = Geo::LPR;
  constexpr int KSTEPS = Geo::KSTEPS, DB = Geo::DB;
  const int4 wk = a.work[blockIdx.x];
  if (wk.x < 0) return;
  const AttnSeq S = a.seqs[wk.x];
  const int c = wk.y, qb = wk.z, sp = wk.w;
  const int G = a.hq / a.hkv;
  const int nq = G * S.M;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  // block qb holds query rows [qb*qbr, qb*qbr + qbr) of the KV head; a wave whose 32 rows are
  // outside the block or all past the end only helps stage the tiles
  const int qbr = S.qrows > 0 ? S.qrows : QB;
  const int t = qb * qbr + wave * 32 + l32;
  const bool wactive = wave * 32 < qbr && qb * qbr + wave * 32 < nq;
  const bool tvalid = wactive && t < nq;
  const int tt = tvalid ? t : nq - 1;
  const int row = S.row_off + tt / G;
  const int h = c * G + tt % G;
  const int k0 = sp * S.chunk;
  const int k1 = min(S.ctx, k0 + S.chunk);
  const int ntiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;

  // this lane's query row as the B operand of S^T = K Q^T: 8 K-steps of 16 dh
  const bf16* qp = (const bf16*)a.Q + ((size_t)row * a.hq + h) * DH + hi * 8;
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);

  __shared__ __attribute__((aligned(1024))) unsigned char kring[NR][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vring[NR][TILE_BYTES];

  // Loads: a tile is TB/1024 chunks of 1 KB (1024/ROWB keys each) of K and as many of V;
  // wave w moves chunks w, w + 8, ... of each.  Lane -> key (1024/ROWB)*chunk + lane/LPR of the
  // tile, LDS slot lane%LPR <- global 16-byte chunk slot ^ swz(key) (swz_k for K, swz_v for
  // V).  The loads are range-checked buffer loads whose resource starts at the tile's first key
  // and ends at the sequence's last cached key: keys past the cache read as zeros (their
  // scores are masked), and the per-lane byte offsets stay the same for every tile.
  int kvo[CPW], vvo[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int kk = (1024 / ROWB) * (wave + 8 * j) + lane / LPR;
    kvo[j] = kk * ROWB + 16 * ((lane % LPR) ^ Geo::swz_k(kk));
    vvo[j] = kk * ROWB + 16 * ((lane % LPR) ^ Geo::swz_v(kk));
  }
  const char* khead = (const char*)S.k + (size_t)c * S.cap * ROWB;
  const char* vhead = (const char*)S.v + (size_t)c * S.cap * ROWB;
  auto tile_rsrc = [&](const char* head, int tile) {
    const int key0 = k0 + tile * KT;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(head + (size_t)key0 * ROWB), (short)0,
                                             (S.ctx - key0) * ROWB, 0x00020000);
  };
  // one tile is staged through registers: loaded in one iteration, stored to LDS in the next
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 stg[2 * CPW];  // this lane's K (0 .. CPW-1) and V (CPW ..) chunks of the staged tile
  auto load_tile = [&](int tile) {
    if (tile >= ntiles) return;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(khead, tile);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vhead, tile);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      stg[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, kvo[j], 0, 0);
      stg[CPW + j] = __builtin_amdgcn_raw_buffer_load_b128(rv, vvo[j], 0, 0);
    }
  };
  auto store_tile = [&](int tile, int slot) {
    if (tile >= ntiles) return;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      *(u32x4*)&kring[slot][(wave + 8 * j) * 1024 + lane * 16] = stg[j];
      *(u32x4*)&vring[slot][(wave + 8 * j) * 1024 + lane * 16] = stg[CPW + j];
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // q arrives scaled by log2(e)/sqrt(dh), so q.k is in the exponent's units.  m: the
  // reference (shared by lanes l, l^32), -inf until the first tile sets it; negm = -m in every
  // entry is the C operand of the first score MFMA of a tile, so the accumulators come out as
  // q.k - m and p = 2^(accumulator) with no per-score shift
  float m = -INFINITY, lsum = 0.f;
  f32x16 negm;
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = 0.f;

  // Loop-invariant LDS byte offsets within a slot.  K read for K-step ks of key l32 (+32 per
  // key block): chunk 2ks + hi in slot chunk ^ swz_k(key).  V^T read (transposing) of lane
  // (g = lane/16, e = (lane/4)%4, q = lane%4) for dh block db: key 4*(g/2) + e (+ the key
  // offset of the MFMA step, a multiple of 8, which leaves swz_v unchanged), dh
  // 32db + 16(g%2) + 4q, i.e. chunk 4db + 2(g%2) + q/2, half q%2, slot chunk ^ swz_v(key).
  int koff[KSTEPS], voff[DB];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    koff[ks] = l32 * ROWB + 16 * ((2 * ks + hi) ^ Geo::swz_k(l32));
  {
    const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
    const int key = 4 * (tg >> 1) + te;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = 4 * db + 2 * (tg & 1) + (tq >> 1);
      voff[db] = key * ROWB + 16 * (ch ^ Geo::swz_v(key)) + 8 * (tq & 1);
    }
  }
  bf16x2 ones2;
  ones2[0] = (bf16)1.f;
  ones2[1] = (bf16)1.f;

  // Per-lane LDS addresses of the V reads in slot 0 of the V ring.  The ring sits above
  // 64 KB, past the reach of the 16-bit instruction offset, so the ring base is folded into
  // the (opaque) register once and slot, key-group and half offsets stay immediates.
  const lds_u8* vbase[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    unsigned a32 = (unsigned)(size_t)(const lds_u8*)&vring[0][0] + (unsigned)voff[db];
    asm volatile("" : "+v"(a32));
    vbase[db] = (const lds_u8*)(size_t)a32;
  }
  // P.V of group g (keys 16g .. 16g+15 of the tile) for the 32-row dh blocks; J = slot
  auto pv_group = [&](int J, int g, const bf16x8& pf) {
    const int kofs = J * TILE_BYTES + ((g >> 1) * 32 + 16 * (g & 1)) * ROWB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const s16x4 lo = lds_read_tr16(vbase[db] + kofs);
      const s16x4 hv = lds_read_tr16(vbase[db] + kofs + 8 * ROWB);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hv, 0, 1, 2, 3, 4, 5, 6, 7));
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
    }
  };
  // scores of the K-steps of group g (KSTEPS/4 of them) for both 32-key blocks; the first
  // K-step starts from -m
  auto qk_steps = [&](const unsigned char* kst, int g, f32x16 (&sc)[2]) {
    constexpr int PER = KSTEPS / 4;
#pragma unroll
    for (int ks = PER * g; ks < PER * g + PER; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(kst + koff[ks] + kb * 32 * ROWB);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], ks == 0 ? negm : sc[kb], 0, 0, 0);
      }
  };
  // probabilities of group g (scores already less the reference); lane holds keys
  // 8*(r/4) + 4*hi + r%4 of the 32-key block g/2, r = 8*(g%2) .. +7; returns their sum (of the
  // rounded values)
  auto probs = [&](const f32x16 (&sc)[2], int g, bf16x8& pf) {
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = (bf16)__builtin_amdgcn_exp2f(sc[g >> 1][8 * (g & 1) + e]);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      bf16x2 pp;
      pp[0] = pf[e];
      pp[1] = pf[e + 1];
      l = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, l, false);
    }
    return l;
  };

  // One tile of the software pipeline; J = it % NR is a compile-time constant so every LDS
  // address is a per-lane register plus an immediate.  Tile t lives in kring/vring[t % NR];
  // iteration it reads K(it+1) and V(it), stores the staged tile it+2 into the slot of tile
  // it-2 (last read in iteration it-2) and loads tile it+3 into the staging registers.
  auto step = [&](auto Jc, int it, f32x16 (&scur)[2], f32x16 (&snext)[2]) {
    constexpr int J = decltype(Jc)::value;
    attn_wait_lgkm0();                       // this wave's LDS stores of the last iteration
    asm volatile("s_barrier" ::: "memory");  // ... and everyone's: K(it+1), V(it) visible
    attn_wait_vmcnt(0);                      // the staged tile it+2 arrived
    store_tile(it + 2, (J + 2) % NR);
    load_tile(it + 3);
    if (!wactive) return;
    const int kt = k0 + it * KT;
    if (kt + KT > k1) {  // ragged last tile (uniform branch)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= k1) scur[kb][r] = -INFINITY;
        }
    }
    float mt = scur[0][0];  // the tile's largest score less the reference
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, scur[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, scur[1][r]);
    mt = pair_max(mt);
    float delta = 0.f;  // raise of the reference (all lanes alike where it is zero)
    if (it == 0) {      // the first tile sets the reference to its largest score
      delta = mt;
      m = mt;
    } else if (__builtin_amdgcn_ballot_w64(mt > RESCALE_LOG2) != 0) {  // some p above 2^8
      delta = mt > RESCALE_LOG2 ? mt : 0.f;
      const float corr = __builtin_amdgcn_exp2f(-delta);
      lsum *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= corr;
      m += delta;
    }
    if (__builtin_amdgcn_ballot_w64(delta != 0.f) != 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        negm[r] = -m;
        scur[0][r] -= delta;
        scur[1][r] -= delta;
      }
    }
    // K(it+1) is stale past the last tile; those scores are never used
    const unsigned char* kst = &kring[(J + 1) % NR][0];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      qk_steps(kst, g, snext);
      bf16x8 pf;
      lsum += probs(scur, g, pf);
      pv_group(J, g, pf);
    }
  };

  f32x16 sa[2], sb[2];
  if (ntiles > 0) {
    load_tile(0);
    attn_wait_vmcnt(0);
    store_tile(0, 0);
    load_tile(1);
    attn_wait_vmcnt(0);
    store_tile(1, 1);
    load_tile(2);
    attn_wait_lgkm0();
    asm volatile("s_barrier" ::: "memory");  // tiles 0 and 1 in LDS
    if (wactive) {
#pragma unroll
      for (int g = 0; g < 4; ++g) qk_steps(&kring[0][0], g, sa);
    }
  }
  static_assert(NR == 4, "the main loop is unrolled by the ring size");
  for (int it = 0; it < ntiles; it += NR) {
    step(std::integral_constant<int, 0>{}, it, sa, sb);
    if (it + 1 >= ntiles) break;
    step(std::integral_constant<int, 1>{}, it + 1, sb, sa);
    if (it + 2 >= ntiles) break;
    step(std::integral_constant<int, 2>{}, it + 2, sa, sb);
    if (it + 3 >= ntiles) break;
    step(std::integral_constant<int, 3>{}, it + 3, sb, sa);
  }
  lsum = pair_sum(lsum);
  if (!tvalid) return;
  const size_t slot = attn_slot(S, sp, tt / G, a.hq, h);
  float* op = a.Opart + slot * DH;
  // O^T accumulator: lane holds dh = 32*db + 8*(r/4) + 4*hi + r%4 of query l32
#pragma unroll
  for (int db = 0; db < DB; ++db) {
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
    a.Mpart[slot] = m;  // log2 domain, like the combine kernel expects
    a.Lpart[slot] = lsum;
  }
}

// ------------------------------------------------------------------------------------
// combine: one wave per (row, query head).  All maxima are in the log2 domain.
// ------------------------------------------------------------------------------------
constexpr int CMB_SPLITS = 32;  // splits whose partial rows are all requested at once

template <class T, int DH, int WK>  // WK: largest window token count of the launch (1 or 8)
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int EPL = DH / 64;  // consecutive dh elements per lane
  // wave-uniform: the row's metadata come through scalar loads
  const int widx = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (widx >= a.R * a.hq) return;
  const int lane = threadIdx.x & 63;
  const int r = widx / a.hq, h = widx % a.hq;
  const int G = a.hq / a.hkv;
  const int c = h / G;
  const AttnSeq S = a.seqs[a.row_seq[r]];
  if (r - S.row_off >= S.M) return;  // a row past the live rows of a live-row plan
  const int e0 = lane * EPL;
  const int rl = r - S.row_off;
  const size_t slot0 = attn_slot(S, 0, rl, a.hq, h);
  const size_t split_stride = (size_t)S.M * a.hq;
  const int ns = S.nsplit;
  // Loads in the order they are needed, all issued before the first wait: the query and the
  // own keys, the splits' (max, denominator), the own values, then the splits' partial rows.
  // window keys: the own keys of the rows of window tokens 0..tw of this state (tw = 0: the
  // row's own key only)
  const int tw = WK == 1 ? 0 : a.row_tok[r];
  const T* q = (const T*)a.Q + ((size_t)r * a.hq + h) * DH + e0;
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = to_f32(q[e]);
  float kw[WK][EPL], vw[WK][EPL];
#pragma unroll
  for (int k = 0; k < WK; ++k)
    if (k <= tw) {
      const float* ks = a.kself + ((size_t)(r - tw + k) * a.hkv + c) * DH + e0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) kw[k][e] = ks[e];
    }
  // lane sp < nsplit holds split sp's (max, denominator); weights 2^(m_sp - M)
  const bool has = lane < ns;
  float m_ld = -INFINITY, l_ld = 0.f;
  if (ns > 0) {  // no splits (an empty cache): no partial slots either
    const size_t lslot = slot0 + (size_t)min(lane, ns - 1) * split_stride;
    m_ld = a.Mpart[lslot];
    l_ld = a.Lpart[lslot];
  }
#pragma unroll
  for (int k = 0; k < WK; ++k)
    if (k <= tw) {
      const float* vs = a.vself + ((size_t)(r - tw + k) * a.hkv + c) * DH + e0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) vw[k][e] = vs[e];
    }
  // the partial rows of the first CMB_SPLITS splits: whole groups of 8, a group's missing
  // splits reading the group's last one (zeroed when added)
  const float* op = a.Opart + slot0 * DH + e0;
  float v[CMB_SPLITS][EPL];
#pragma unroll
  for (int g = 0; g < CMB_SPLITS / 8; ++g) {
    if (8 * g >= ns) break;
#pragma unroll
    for (int j = 8 * g; j < 8 * g + 8; ++j) {
      const float* pj = op + (size_t)min(j, ns - 1) * split_stride * DH;
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[j][e] = pj[e];
    }
  }

  float s_w[WK];
#pragma unroll
  for (int k = 0; k < WK; ++k) {
    s_w[k] = -INFINITY;
    if (k <= tw) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qv[e], kw[k][e], d);
      s_w[k] = warp_sum(d) * a.scale_log2;
    }
  }
  const size_t qrow = (size_t)r * a.hq + h;
  const float ms = has ? m_ld : -INFINITY;
  const float ls = has ? l_ld : 0.f;
  float mx = fmaxf(warp_max(ms), s_w[0]);
#pragma unroll
  for (int k = 1; k < WK; ++k)
    if (k <= tw) mx = fmaxf(mx, s_w[k]);
  const float wsp = has ? exp2f(ms - mx) : 0.f;
  float w_w[WK];
#pragma unroll
  for (int k = 0; k < WK; ++k) w_w[k] = k <= tw ? exp2f(s_w[k] - mx) : 0.f;
  float den = warp_sum(wsp * ls) + w_w[0];
#pragma unroll
  for (int k = 1; k < WK; ++k)
    if (k <= tw) den += w_w[k];
  const float inv = 1.0f / den;
  float num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = w_w[0] * vw[0][e];
#pragma unroll
  for (int k = 1; k < WK; ++k) {
    if (k <= tw) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) num[e] = fmaf(w_w[k], vw[k][e], num[e]);
    }
  }
  // splits added in order, in groups of 8 (a group's missing splits add 0 * 0)
#pragma unroll
  for (int g = 0; g < CMB_SPLITS / 8; ++g) {
    if (8 * g >= ns) break;
#pragma unroll
    for (int j = 8 * g; j < 8 * g + 8; ++j) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsp), j));
#pragma unroll
      for (int e = 0; e < EPL; ++e) num[e] = fmaf(w, j < ns ? v[j][e] : 0.f, num[e]);
    }
  }
  // splits past CMB_SPLITS (at most 64, one per lane), 8 at a time
  for (int sp0 = CMB_SPLITS; sp0 < ns; sp0 += 8) {
    float u[8][EPL];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* pj = op + (size_t)(sp0 + j) * split_stride * DH;
#pragma unroll
      for (int e = 0; e < EPL; ++e) u[j][e] = sp0 + j < ns ? pj[e] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsp), min(sp0 + j, 63)));
#pragma unroll
      for (int e = 0; e < EPL; ++e) num[e] = fmaf(w, u[j][e], num[e]);
    }
  }
  T* out = (T*)a.O + qrow * DH + e0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = from_f32<T>(num[e] * inv);
}

template <class T>
__global__ __launch_bounds__(256) void kv_append_kernel(const float* kself, const float* vself,
                                                       int n, int hkv, int dh, T* kc, T* vc,
                                                       int cap, int pos0) {
  const size_t total = (size_t)n * hkv * dh;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int e = (int)(i % dh);
  const int c = (int)((i / dh) % hkv);
  const int t = (int)(i / ((size_t)dh * hkv));
  const size_t dst = ((size_t)c * cap + pos0 + t) * dh + e;
  kc[dst] = from_f32<T>(kself[i]);
  vc[dst] = from_f32<T>(vself[i]);
}

}  // namespace

// bfloat16 at head size 64 or 128 runs the MFMA kernel, everything else the VALU kernel
static bool mfma_path(int act, int dh) { return act == ACT_BF16 && (dh == 128 || dh == 64); }
int attention_qblock(int act, int dh) { return mfma_path(act, dh) ? QB : 64; }
// MFMA kernel: 64 KB (DH 64) or 128 KB (DH 128) of LDS rings and 512 threads -> one per CU;
// VALU kernel: 64 threads, <= 33 KB LDS
int attention_wgs_per_cu(int act, int dh) { return mfma_path(act, dh) ? 1 : 4; }

hipError_t launch_qkv(const QkvArgs& a, int act, hipStream_t s) {
  if (a.splits < 1 || a.splits > GEMM_MAX_SPLITS || a.dh > 128) return hipErrorInvalidValue;
  const int waves = a.R * (a.hq + 2 * a.hkv);
  const dim3 grid((waves + 3) / 4), block(256);
  if (act == ACT_F32)
    hipLaunchKernelGGL(qkv_kernel<float>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(qkv_kernel<bf16>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const float* kself, const float* vself, int n, int hkv, int dh,
                            void* kc, void* vc, int cap, int pos0, int act, hipStream_t s) {
  const size_t total = (size_t)n * hkv * dh;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (act == ACT_F32)
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, block, 0, s, kself, vself, n, hkv, dh,
                       (float*)kc, (float*)vc, cap, pos0);
  else
    hipLaunchKernelGGL(kv_append_kernel<bf16>, grid, block, 0, s, kself, vself, n, hkv, dh,
                       (bf16*)kc, (bf16*)vc, cap, pos0);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int act, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  if (act == ACT_BF16) {
    if (a.dh == 128)
      hipLaunchKernelGGL(attn_mfma_kernel<128>, dim3(n_work), dim3(512), 0, s, a);
    else if (a.dh == 64)
      hipLaunchKernelGGL(attn_mfma_kernel<64>, dim3(n_work), dim3(512), 0, s, a);
    else
      return hipErrorInvalidValue;
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

template <class T, int DH>
static void launch_combine_t(const CombineArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.rmax > 1)
    hipLaunchKernelGGL((combine_kernel<T, DH, WIN_MAX>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<T, DH, 1>), grid, block, 0, s, a);
}

hipError_t launch_combine(const CombineArgs& a, int act, hipStream_t s) {
  const int waves = a.R * a.hq;
  const dim3 grid((waves + 3) / 4), block(256);
  if (a.dh != 64 && a.dh != 128) return hipErrorInvalidValue;
  if (act == ACT_F32) {
    if (a.dh == 64)
      launch_combine_t<float, 64>(a, grid, block, s);
    else
      launch_combine_t<float, 128>(a, grid, block, s);
  } else {
    if (a.dh == 64)
      launch_combine_t<bf16, 64>(a, grid, block, s);
    else
      launch_combine_t<bf16, 128>(a, grid, block, s);
  }
  return hipGetLastError();
}

}  // namespace ks
