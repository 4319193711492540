// Per-budget execute/skip select of the KnapSpec DP and the DP's initial state.
//
// reduce_rows: the item's GEMM wrote fp32 K-split partials of F_i(x) - x for each source row
// and the reference row; one fully parallel pass adds the splits (fixed order) and the
// residual, E[r] = x_src(r) + dF(r).
// select: one workgroup per (sequence, budget b) and one per sequence for the reference; it
// forms
//   c_exec = cos(E[row of b - w_i], ref'),   c_skip = cos(g[b], ref'),   ref' = E[ref row],
// keeps the larger (skip on exact ties, NaN as -inf), applies the tau / skip-cap pruning,
// carries the layer mask, and writes the kept state together with its RMSNorm'd copy in the
// activation layout of the next item's GEMM (so the norm is fused into the select).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ks {

namespace {

constexpr int SEL_THREADS = 256;
constexpr int SELR_THREADS = 512;  // register-resident select: up to SELR_MAXIT float4 per row
constexpr int SELR_MAXIT = 4;

__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  const int d4 = a.d / 4;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)a.R * d4) return;
  const int r = (int)(idx / d4), e4 = (int)(idx % d4);
  const size_t split_stride = (size_t)a.R * a.d;
  const size_t off = (size_t)r * a.d + 4 * e4;
  const f32x4 res = *(const f32x4*)(a.state_old + (size_t)a.row_state[r] * a.d + 4 * e4);
  // every split's load in flight before the first addition; the sum keeps the split order
  f32x4 p[GEMM_MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < GEMM_MAX_SPLITS; ++s)
    if (s < a.splits) p[s] = *(const f32x4*)(a.P + s * split_stride + off);
  f32x4 v = p[0];
#pragma unroll
  for (int s = 1; s < GEMM_MAX_SPLITS; ++s)
    if (s < a.splits) v += p[s];
  *(f32x4*)(a.E + off) = res + v;
}

template <int N, int THREADS = SEL_THREADS>
__device__ __forceinline__ void block_sum(float (&v)[N], float* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = warp_sum(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) scratch[wave * N + i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float t = scratch[i];
    for (int w = 1; w < THREADS / 64; ++w) t += scratch[w * N + i];
    v[i] = t;
  }
  __syncthreads();
}

template <class T>
__device__ __forceinline__ void store_act(void* xa, size_t row, int d, int e4, f32x4 x,
                                          float scale) {
  T* p = (T*)xa + row * d + 4 * e4;
  p[0] = from_f32<T>(x[0] * scale);
  p[1] = from_f32<T>(x[1] * scale);
  p[2] = from_f32<T>(x[2] * scale);
  p[3] = from_f32<T>(x[3] * scale);
}

__device__ __forceinline__ float nan_to_ninf(float c) { return (c == c) ? c : -INFINITY; }

template <class T>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(SelectArgs a) {
  const int q = blockIdx.x / (a.B + 1);
  const int b = blockIdx.x % (a.B + 1);
  const bool is_ref = b == a.B;
  const ItemSeq inf = a.info[q];
  const int d4 = a.d / 4;
  const size_t slot = (size_t)a.kmax * a.wmax * a.d;  // floats per budget slot (token 0 used)
  const size_t sstride = (size_t)(a.Bm + 1) * slot;  // per-sequence state stride
  const float* st_old = a.state_old + q * sstride;
  float* st_new = a.state_new + q * sstride;
  const float* ref = a.E + (size_t)inf.ref_row * a.d;
  __shared__ float scratch[8 * (SEL_THREADS / 64)];

  if (is_ref) {
    float ss[1] = {0.f};
    for (int e4 = threadIdx.x; e4 < d4; e4 += SEL_THREADS) {
      const f32x4 r = *(const f32x4*)(ref + 4 * e4);
      *(f32x4*)(st_new + (size_t)a.Bm * slot + 4 * e4) = r;
      ss[0] += r[0] * r[0] + r[1] * r[1] + r[2] * r[2] + r[3] * r[3];
    }
    if (inf.next_ref_row < 0) return;
    block_sum<1>(ss, scratch);
    const float scale = 1.0f / sqrtf(ss[0] / (float)a.d + a.eps);
    for (int e4 = threadIdx.x; e4 < d4; e4 += SEL_THREADS) {
      const f32x4 r = *(const f32x4*)(st_new + (size_t)a.Bm * slot + 4 * e4);
      store_act<T>(a.xa_next, inf.next_ref_row, a.d, e4, r, scale);
    }
    return;
  }

  const int qb = q * a.Bm + b;
  const int erow = a.exec_row[(size_t)qb * a.kmax];
  const int src = b - inf.w;
  const bool has_exec = erow >= 0 && src >= 0 && a.valid_old[(size_t)(q * a.Bm + src) * a.kmax];
  const bool has_skip = a.valid_old[(size_t)qb * a.kmax] != 0;
  const float* e_row = a.E + (size_t)(has_exec ? erow : 0) * a.d;
  const float* g_row = st_old + (size_t)b * slot;

  // pass 1: rr, er, ee, gr, gg
  float acc[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
  if (has_exec || has_skip) {
    for (int e4 = threadIdx.x; e4 < d4; e4 += SEL_THREADS) {
      const f32x4 r = *(const f32x4*)(ref + 4 * e4);
      acc[0] += r[0] * r[0] + r[1] * r[1] + r[2] * r[2] + r[3] * r[3];
      if (has_exec) {
        const f32x4 ev = *(const f32x4*)(e_row + 4 * e4);
        acc[1] += ev[0] * r[0] + ev[1] * r[1] + ev[2] * r[2] + ev[3] * r[3];
        acc[2] += ev[0] * ev[0] + ev[1] * ev[1] + ev[2] * ev[2] + ev[3] * ev[3];
      }
      if (has_skip) {
        const f32x4 gv = *(const f32x4*)(g_row + 4 * e4);
        acc[3] += gv[0] * r[0] + gv[1] * r[1] + gv[2] * r[2] + gv[3] * r[3];
        acc[4] += gv[0] * gv[0] + gv[1] * gv[1] + gv[2] * gv[2] + gv[3] * gv[3];
      }
    }
  }
  block_sum<5>(acc, scratch);
  const float c_e = has_exec ? nan_to_ninf(acc[1] / (sqrtf(acc[2]) * sqrtf(acc[0]))) : -INFINITY;
  const float c_s = has_skip ? nan_to_ninf(acc[3] / (sqrtf(acc[4]) * sqrtf(acc[0]))) : -INFINITY;
  const bool take = c_e > c_s;
  const float best = take ? c_e : c_s;
  bool alive = best > -INFINITY;
  if (best < a.tau) alive = false;
  if (a.skip_cap >= 0 && inf.prefix - b > a.skip_cap) alive = false;

  if (threadIdx.x == 0) {
    a.valid_new[(size_t)qb * a.kmax] = alive ? 1 : 0;
    const size_t cell = ((size_t)q * a.n_items + a.item) * a.Bm + b;
    if (a.decisions) a.decisions[cell] = alive ? (take ? 1 : 0) : 255;
    if (a.margins) {
      const bool he = c_e > -INFINITY, hs = c_s > -INFINITY;
      a.margins[cell] = (he && hs) ? fabsf(c_e - c_s) : ((he != hs) ? INFINITY : NAN);
    }
    if (a.item == a.n_items - 1) a.cos_out[qb] = alive ? best : NAN;
  }
  if (threadIdx.x < a.mw) {
    const int wd = threadIdx.x;
    uint64_t mval = 0;
    if (alive) {
      if (take) {
        mval = a.mask_old[((size_t)q * a.Bm + src) * a.kmax * a.mw + wd];
        if (wd == a.item / 64) mval |= (uint64_t)1 << (a.item % 64);
      } else {
        mval = a.mask_old[(size_t)qb * a.kmax * a.mw + wd];
      }
    }
    a.mask_new[(size_t)qb * a.kmax * a.mw + wd] = mval;
  }

  // pass 2: kept state and its RMSNorm'd activation row for the next item
  const int nrow = a.next_row[(size_t)qb * a.kmax];
  if (!alive) {
    if (nrow >= 0) {
      for (int e4 = threadIdx.x; e4 < d4; e4 += SEL_THREADS) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        store_act<T>(a.xa_next, nrow, a.d, e4, z, 0.f);
      }
    }
    return;
  }
  const float ms = (take ? acc[2] : acc[4]) / (float)a.d;
  const float scale = 1.0f / sqrtf(ms + a.eps);
  float* out = st_new + (size_t)b * slot;
  for (int e4 = threadIdx.x; e4 < d4; e4 += SEL_THREADS) {
    const f32x4 x = take ? *(const f32x4*)(e_row + 4 * e4) : *(const f32x4*)(g_row + 4 * e4);
    *(f32x4*)(out + 4 * e4) = x;
    if (nrow >= 0) store_act<T>(a.xa_next, nrow, a.d, e4, x, scale);
  }
}

// The same select with the rows held in registers between the two passes (one global read of
// each row instead of two) and 512 threads per budget: for d <= 4 * 4 * SELR_THREADS and
// single-token states (window r = 1; a budget's state is token 0 of its wmax-row slot).
// Sums are taken in the same per-thread order as select_kernel would with 512 threads; the
// decision and the written rows are those of the definition above.
template <class T, int IT>
__global__ __launch_bounds__(SELR_THREADS) void select_reg_kernel(SelectArgs a) {
  const int q = blockIdx.x / (a.B + 1);
  const int b = blockIdx.x % (a.B + 1);
  const bool is_ref = b == a.B;
  const ItemSeq inf = a.info[q];
  const int d4 = a.d / 4;
  const size_t slot = (size_t)a.kmax * a.wmax * a.d;  // floats per budget slot
  const size_t sstride = (size_t)(a.Bm + 1) * slot;
  const float* st_old = a.state_old + q * sstride;
  float* st_new = a.state_new + q * sstride;
  const float* ref = a.E + (size_t)inf.ref_row * a.d;
  __shared__ float scratch[8 * (SELR_THREADS / 64)];
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  if (is_ref) {
    f32x4 r[IT];
    float ss[1] = {0.f};
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int e4 = threadIdx.x + i * SELR_THREADS;
      r[i] = e4 < d4 ? *(const f32x4*)(ref + 4 * e4) : zero;
      if (e4 < d4) *(f32x4*)(st_new + (size_t)a.Bm * slot + 4 * e4) = r[i];
      ss[0] += r[i][0] * r[i][0] + r[i][1] * r[i][1] + r[i][2] * r[i][2] + r[i][3] * r[i][3];
    }
    if (inf.next_ref_row < 0) return;
    block_sum<1, SELR_THREADS>(ss, scratch);
    const float scale = 1.0f / sqrtf(ss[0] / (float)a.d + a.eps);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int e4 = threadIdx.x + i * SELR_THREADS;
      if (e4 < d4) store_act<T>(a.xa_next, inf.next_ref_row, a.d, e4, r[i], scale);
    }
    return;
  }

  const int qb = q * a.Bm + b;
  const int erow = a.exec_row[(size_t)qb * a.kmax];
  const int src = b - inf.w;
  const float* e_row = a.E + (size_t)(erow >= 0 ? erow : 0) * a.d;
  const float* g_row = st_old + (size_t)b * slot;
  // The validity flags and both candidates' mask words are requested first and the rows right
  // after, without waiting in between (every address is in range); a row that takes no part
  // is replaced by zeros below, as if it had not been read.
  const int v_src = a.valid_old[(size_t)(q * a.Bm + (src >= 0 ? src : 0)) * a.kmax];
  const int v_skip = a.valid_old[(size_t)qb * a.kmax];
  uint64_t mask_exec = 0, mask_skip = 0;
  if (threadIdx.x < a.mw) {
    mask_exec = a.mask_old[((size_t)q * a.Bm + (src >= 0 ? src : 0)) * a.kmax * a.mw + threadIdx.x];
    mask_skip = a.mask_old[(size_t)qb * a.kmax * a.mw + threadIdx.x];
  }
  f32x4 rv[IT], ev[IT], gv[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e4 = threadIdx.x + i * SELR_THREADS;
    const bool in = e4 < d4;
    rv[i] = in ? *(const f32x4*)(ref + 4 * e4) : zero;
    ev[i] = in ? *(const f32x4*)(e_row + 4 * e4) : zero;
    gv[i] = in ? *(const f32x4*)(g_row + 4 * e4) : zero;
  }
  const bool has_exec = erow >= 0 && src >= 0 && v_src != 0;
  const bool has_skip = v_skip != 0;
  const int nrow = a.next_row[(size_t)qb * a.kmax];

  float acc[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const f32x4 r = (has_exec || has_skip) ? rv[i] : zero;
    if (!has_exec) ev[i] = zero;
    if (!has_skip) gv[i] = zero;
    acc[0] += r[0] * r[0] + r[1] * r[1] + r[2] * r[2] + r[3] * r[3];
    acc[1] += ev[i][0] * r[0] + ev[i][1] * r[1] + ev[i][2] * r[2] + ev[i][3] * r[3];
    acc[2] += ev[i][0] * ev[i][0] + ev[i][1] * ev[i][1] + ev[i][2] * ev[i][2] + ev[i][3] * ev[i][3];
    acc[3] += gv[i][0] * r[0] + gv[i][1] * r[1] + gv[i][2] * r[2] + gv[i][3] * r[3];
    acc[4] += gv[i][0] * gv[i][0] + gv[i][1] * gv[i][1] + gv[i][2] * gv[i][2] + gv[i][3] * gv[i][3];
  }
  block_sum<5, SELR_THREADS>(acc, scratch);
  const float c_e = has_exec ? nan_to_ninf(acc[1] / (sqrtf(acc[2]) * sqrtf(acc[0]))) : -INFINITY;
  const float c_s = has_skip ? nan_to_ninf(acc[3] / (sqrtf(acc[4]) * sqrtf(acc[0]))) : -INFINITY;
  const bool take = c_e > c_s;
  const float best = take ? c_e : c_s;
  bool alive = best > -INFINITY;
  if (best < a.tau) alive = false;
  if (a.skip_cap >= 0 && inf.prefix - b > a.skip_cap) alive = false;

  if (threadIdx.x == 0) {
    a.valid_new[(size_t)qb * a.kmax] = alive ? 1 : 0;
    const size_t cell = ((size_t)q * a.n_items + a.item) * a.Bm + b;
    if (a.decisions) a.decisions[cell] = alive ? (take ? 1 : 0) : 255;
    if (a.margins) {
      const bool he = c_e > -INFINITY, hs = c_s > -INFINITY;
      a.margins[cell] = (he && hs) ? fabsf(c_e - c_s) : ((he != hs) ? INFINITY : NAN);
    }
    if (a.item == a.n_items - 1) a.cos_out[qb] = alive ? best : NAN;
  }
  if (threadIdx.x < a.mw) {
    const int wd = threadIdx.x;
    uint64_t mval = 0;
    if (alive) {
      if (take) {
        mval = mask_exec;
        if (wd == a.item / 64) mval |= (uint64_t)1 << (a.item % 64);
      } else {
        mval = mask_skip;
      }
    }
    a.mask_new[(size_t)qb * a.kmax * a.mw + wd] = mval;
  }

  const float ms = (take ? acc[2] : acc[4]) / (float)a.d;
  const float scale = alive ? 1.0f / sqrtf(ms + a.eps) : 0.f;
  float* out = st_new + (size_t)b * slot;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e4 = threadIdx.x + i * SELR_THREADS;
    if (e4 >= d4) continue;
    const f32x4 x = alive ? (take ? ev[i] : gv[i]) : zero;
    if (alive) *(f32x4*)(out + 4 * e4) = x;
    if (nrow >= 0) store_act<T>(a.xa_next, nrow, a.d, e4, x, scale);
  }
}

// Select for r-token states (window r = ItemSeq::win, 1..WIN_MAX): the cosine is taken over
// the flattened r x d state (sums over all r rows), the decision is the one above, and each
// kept token row gets its own RMSNorm scale for the next item's activations.  Two passes
// over the rows (the second re-reads the kept rows).
constexpr int SELW_THREADS = 512;
constexpr int SELW_SUMS = 5 + 2 * WIN_MAX;  // rr, er, ee, gr, gg, ee_t[r], gg_t[r]

template <class T>
__global__ __launch_bounds__(SELW_THREADS) void select_win_kernel(SelectArgs a) {
  const int q = blockIdx.x / (a.B + 1);
  const int b = blockIdx.x % (a.B + 1);
  const bool is_ref = b == a.B;
  const ItemSeq inf = a.info[q];
  const int r = inf.win;
  const int d4 = a.d / 4;
  const size_t slot = (size_t)a.kmax * a.wmax * a.d;
  const size_t sstride = (size_t)(a.Bm + 1) * slot;
  const float* st_old = a.state_old + q * sstride;
  float* st_new = a.state_new + q * sstride;
  const float* ref = a.E + (size_t)inf.ref_row * a.d;  // r consecutive rows
  __shared__ float scratch[SELW_SUMS * (SELW_THREADS / 64)];

  if (is_ref) {
    float ss[WIN_MAX];
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) ss[t] = 0.f;
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) {
      if (t >= r) continue;
      for (int e4 = threadIdx.x; e4 < d4; e4 += SELW_THREADS) {
        const f32x4 x = *(const f32x4*)(ref + (size_t)t * a.d + 4 * e4);
        *(f32x4*)(st_new + (size_t)a.Bm * slot + (size_t)t * a.d + 4 * e4) = x;
        ss[t] += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
      }
    }
    if (inf.next_ref_row < 0) return;
    block_sum<WIN_MAX, SELW_THREADS>(ss, scratch);
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) {
      if (t >= r) continue;
      const float scale = 1.0f / sqrtf(ss[t] / (float)a.d + a.eps);
      for (int e4 = threadIdx.x; e4 < d4; e4 += SELW_THREADS) {
        const f32x4 x = *(const f32x4*)(st_new + (size_t)a.Bm * slot + (size_t)t * a.d + 4 * e4);
        store_act<T>(a.xa_next, inf.next_ref_row + t, a.d, e4, x, scale);
      }
    }
    return;
  }

  const int qb = q * a.Bm + b;
  const int erow = a.exec_row[(size_t)qb * a.kmax];
  const int src = b - inf.w;
  const bool has_exec = erow >= 0 && src >= 0 && a.valid_old[(size_t)(q * a.Bm + src) * a.kmax];
  const bool has_skip = a.valid_old[(size_t)qb * a.kmax] != 0;
  const float* e_row = a.E + (size_t)(has_exec ? erow : 0) * a.d;  // r consecutive rows
  const float* g_row = st_old + (size_t)b * slot;                    // r rows of the slot

  float acc[SELW_SUMS];
#pragma unroll
  for (int i = 0; i < SELW_SUMS; ++i) acc[i] = 0.f;
  if (has_exec || has_skip) {
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) {
      if (t >= r) continue;
      for (int e4 = threadIdx.x; e4 < d4; e4 += SELW_THREADS) {
        const size_t o = (size_t)t * a.d + 4 * e4;
        const f32x4 rv = *(const f32x4*)(ref + o);
        acc[0] += rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2] + rv[3] * rv[3];
        if (has_exec) {
          const f32x4 ev = *(const f32x4*)(e_row + o);
          acc[1] += ev[0] * rv[0] + ev[1] * rv[1] + ev[2] * rv[2] + ev[3] * rv[3];
          const float ee = ev[0] * ev[0] + ev[1] * ev[1] + ev[2] * ev[2] + ev[3] * ev[3];
          acc[2] += ee;
          acc[5 + t] += ee;
        }
        if (has_skip) {
          const f32x4 gv = *(const f32x4*)(g_row + o);
          acc[3] += gv[0] * rv[0] + gv[1] * rv[1] + gv[2] * rv[2] + gv[3] * rv[3];
          const float gg = gv[0] * gv[0] + gv[1] * gv[1] + gv[2] * gv[2] + gv[3] * gv[3];
          acc[4] += gg;
          acc[5 + WIN_MAX + t] += gg;
        }
      }
    }
  }
  block_sum<SELW_SUMS, SELW_THREADS>(acc, scratch);
  const float c_e = has_exec ? nan_to_ninf(acc[1] / (sqrtf(acc[2]) * sqrtf(acc[0]))) : -INFINITY;
  const float c_s = has_skip ? nan_to_ninf(acc[3] / (sqrtf(acc[4]) * sqrtf(acc[0]))) : -INFINITY;
  const bool take = c_e > c_s;
  const float best = take ? c_e : c_s;
  bool alive = best > -INFINITY;
  if (best < a.tau) alive = false;
  if (a.skip_cap >= 0 && inf.prefix - b > a.skip_cap) alive = false;

  if (threadIdx.x == 0) {
    a.valid_new[(size_t)qb * a.kmax] = alive ? 1 : 0;
    const size_t cell = ((size_t)q * a.n_items + a.item) * a.Bm + b;
    if (a.decisions) a.decisions[cell] = alive ? (take ? 1 : 0) : 255;
    if (a.margins) {
      const bool he = c_e > -INFINITY, hs = c_s > -INFINITY;
      a.margins[cell] = (he && hs) ? fabsf(c_e - c_s) : ((he != hs) ? INFINITY : NAN);
    }
    if (a.item == a.n_items - 1) a.cos_out[qb] = alive ? best : NAN;
  }
  if (threadIdx.x < a.mw) {
    const int wd = threadIdx.x;
    uint64_t mval = 0;
    if (alive) {
      if (take) {
        mval = a.mask_old[((size_t)q * a.Bm + src) * a.kmax * a.mw + wd];
        if (wd == a.item / 64) mval |= (uint64_t)1 << (a.item % 64);
      } else {
        mval = a.mask_old[(size_t)qb * a.kmax * a.mw + wd];
      }
    }
    a.mask_new[(size_t)qb * a.kmax * a.mw + wd] = mval;
  }

  const int nrow = a.next_row[(size_t)qb * a.kmax];
  float* out = st_new + (size_t)b * slot;
#pragma unroll
  for (int t = 0; t < WIN_MAX; ++t) {
    if (t >= r) continue;
    const float ms = (take ? acc[5 + t] : acc[5 + WIN_MAX + t]) / (float)a.d;
    const float scale = alive ? 1.0f / sqrtf(ms + a.eps) : 0.f;
    const float* xr = (take ? e_row : g_row) + (size_t)t * a.d;
    for (int e4 = threadIdx.x; e4 < d4; e4 += SELW_THREADS) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 x = alive ? *(const f32x4*)(xr + 4 * e4) : zero;
      if (alive) *(f32x4*)(out + (size_t)t * a.d + 4 * e4) = x;
      if (nrow >= 0) store_act<T>(a.xa_next, nrow + t, a.d, e4, x, scale);
    }
  }
}

// Select of the beam variant (beam k = SelectArgs::beam in 2..BEAM_MAX, any window r): the
// candidates of budget b are its k skip states (slots of b) and the item applied to the k
// states of b - w (rows of this item); each is scored by the cosine of its flattened r x d
// state with the reference, ranked higher first with ties to the lower candidate index
// (skip slots 0..k-1, then execute slots 0..k-1), NaN as -inf; the first k valid candidates
// that pass tau and the skip cap become slots 0..k-1.  Kept rows get per-token RMSNorm scales
// for the next item's activations.
constexpr int SELB_THREADS = 512;
constexpr int SELB_SUMS = 1 + 4 * BEAM_MAX;  // rr, then (dot, norm^2) of 2k candidates

template <class T>
__global__ __launch_bounds__(SELB_THREADS) void select_beam_kernel(SelectArgs a) {
  const int q = blockIdx.x / (a.B + 1);
  const int b = blockIdx.x % (a.B + 1);
  const bool is_ref = b == a.B;
  const ItemSeq inf = a.info[q];
  const int r = inf.win, K = a.beam;
  const int d4 = a.d / 4;
  const size_t bslot = (size_t)a.wmax * a.d;     // floats per beam slot
  const size_t bstride = (size_t)a.kmax * bslot;  // floats per budget
  const size_t sstride = (size_t)(a.Bm + 1) * bstride;
  const float* st_old = a.state_old + q * sstride;
  float* st_new = a.state_new + q * sstride;
  const float* ref = a.E + (size_t)inf.ref_row * a.d;
  __shared__ float scratch[SELB_SUMS * (SELB_THREADS / 64)];
  __shared__ int keep[BEAM_MAX];

  if (is_ref) {
    float ss[WIN_MAX];
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) ss[t] = 0.f;
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) {
      if (t >= r) continue;
      for (int e4 = threadIdx.x; e4 < d4; e4 += SELB_THREADS) {
        const f32x4 x = *(const f32x4*)(ref + (size_t)t * a.d + 4 * e4);
        *(f32x4*)(st_new + (size_t)a.Bm * bstride + (size_t)t * a.d + 4 * e4) = x;
        ss[t] += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
      }
    }
    if (inf.next_ref_row < 0) return;
    block_sum<WIN_MAX, SELB_THREADS>(ss, scratch);
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) {
      if (t >= r) continue;
      const float scale = 1.0f / sqrtf(ss[t] / (float)a.d + a.eps);
      for (int e4 = threadIdx.x; e4 < d4; e4 += SELB_THREADS) {
        const f32x4 x =
            *(const f32x4*)(st_new + (size_t)a.Bm * bstride + (size_t)t * a.d + 4 * e4);
        store_act<T>(a.xa_next, inf.next_ref_row + t, a.d, e4, x, scale);
      }
    }
    return;
  }

  const size_t qbk = ((size_t)q * a.Bm + b) * a.kmax;       // first slot entry of budget b
  const int src = b - inf.w;
  const size_t sbk = ((size_t)q * a.Bm + (src >= 0 ? src : 0)) * a.kmax;
  // candidate c: c < K skip state of slot c; K <= c < 2K item output of source slot c - K
  auto cand_row = [&](int c) -> const float* {
    if (c < K) return st_old + (size_t)b * bstride + (size_t)c * bslot;
    return a.E + (size_t)a.exec_row[qbk + (c - K)] * a.d;
  };
  bool has[2 * BEAM_MAX];
#pragma unroll
  for (int c = 0; c < 2 * BEAM_MAX; ++c) {
    has[c] = false;
    if (c < K) {
      has[c] = a.valid_old[qbk + c] != 0;
    } else if (c < 2 * K) {
      const int j = c - K;
      has[c] = a.exec_row[qbk + j] >= 0 && src >= 0 && a.valid_old[sbk + j] != 0;
    }
  }
  float acc[SELB_SUMS];
#pragma unroll
  for (int i = 0; i < SELB_SUMS; ++i) acc[i] = 0.f;
  for (int t = 0; t < r; ++t) {
    for (int e4 = threadIdx.x; e4 < d4; e4 += SELB_THREADS) {
      const size_t o = (size_t)t * a.d + 4 * e4;
      const f32x4 rv = *(const f32x4*)(ref + o);
      acc[0] += rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2] + rv[3] * rv[3];
#pragma unroll
      for (int c = 0; c < 2 * BEAM_MAX; ++c) {
        if (!has[c]) continue;
        const f32x4 x = *(const f32x4*)(cand_row(c) + o);
        acc[1 + 2 * c] += x[0] * rv[0] + x[1] * rv[1] + x[2] * rv[2] + x[3] * rv[3];
        acc[2 + 2 * c] += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
      }
    }
  }
  block_sum<SELB_SUMS, SELB_THREADS>(acc, scratch);
  if (threadIdx.x == 0) {
    float cs[2 * BEAM_MAX];
    int order[2 * BEAM_MAX];
    int n = 0;
    for (int c = 0; c < 2 * K; ++c) {
      cs[c] = has[c] ? nan_to_ninf(acc[1 + 2 * c] / (sqrtf(acc[2 + 2 * c]) * sqrtf(acc[0])))
                     : -INFINITY;
      // insertion by (cosine descending, candidate index ascending)
      int p = n++;
      while (p > 0 && cs[order[p - 1]] < cs[c]) {
        order[p] = order[p - 1];
        --p;
      }
      order[p] = c;
    }
    const bool capped = a.skip_cap >= 0 && inf.prefix - b > a.skip_cap;
    int kept = 0;
    for (int m = 0; m < n && kept < K && !capped; ++m) {
      const int c = order[m];
      if (!(cs[c] > -INFINITY) || cs[c] < a.tau) break;
      keep[kept++] = c;
    }
    for (int j = kept; j < K; ++j) keep[j] = -1;
    if (a.item == a.n_items - 1) a.cos_out[q * a.Bm + b] = kept ? cs[keep[0]] : NAN;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < a.kmax; j += SELB_THREADS)
    a.valid_new[qbk + j] = (j < K && keep[j] >= 0) ? 1 : 0;
  for (int idx = threadIdx.x; idx < K * a.mw; idx += SELB_THREADS) {
    const int j = idx / a.mw, wd = idx % a.mw;
    const int c = keep[j];
    uint64_t mval = 0;
    if (c >= 0 && c < K) {
      mval = a.mask_old[(qbk + c) * a.mw + wd];
    } else if (c >= K) {
      mval = a.mask_old[(sbk + (c - K)) * a.mw + wd];
      if (wd == a.item / 64) mval |= (uint64_t)1 << (a.item % 64);
    }
    a.mask_new[(qbk + j) * a.mw + wd] = mval;
  }
  // kept states and their RMSNorm'd rows for the next item
  for (int j = 0; j < K; ++j) {
    const int c = keep[j];
    const int nrow = a.next_row[qbk + j];
    if (c < 0) {
      if (nrow >= 0) {
        for (int t = 0; t < r; ++t)
          for (int e4 = threadIdx.x; e4 < d4; e4 += SELB_THREADS) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            store_act<T>(a.xa_next, nrow + t, a.d, e4, z, 0.f);
          }
      }
      continue;
    }
    const float* xr = cand_row(c);
    float* out = st_new + (size_t)b * bstride + (size_t)j * bslot;
    float ss[WIN_MAX];
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) ss[t] = 0.f;
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) {
      if (t >= r) continue;
      for (int e4 = threadIdx.x; e4 < d4; e4 += SELB_THREADS) {
        const f32x4 x = *(const f32x4*)(xr + (size_t)t * a.d + 4 * e4);
        *(f32x4*)(out + (size_t)t * a.d + 4 * e4) = x;
        ss[t] += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
      }
    }
    if (nrow < 0) continue;
    block_sum<WIN_MAX, SELB_THREADS>(ss, scratch);
#pragma unroll
    for (int t = 0; t < WIN_MAX; ++t) {
      if (t >= r) continue;
      const float scale = 1.0f / sqrtf(ss[t] / (float)a.d + a.eps);
      for (int e4 = threadIdx.x; e4 < d4; e4 += SELB_THREADS) {
        const f32x4 x = *(const f32x4*)(xr + (size_t)t * a.d + 4 * e4);
        store_act<T>(a.xa_next, nrow + t, a.d, e4, x, scale);
      }
    }
  }
}

// Greedy-token reduction over one vocabulary chunk: one wave per row.
__global__ __launch_bounds__(256) void lm_argmax_kernel(LmArgmaxArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.R) return;
  const int lane = threadIdx.x & 63;
  const size_t sstride = (size_t)a.R * a.ldp;
  const float* p = a.P + (size_t)row * a.ldp;
  float bv = -INFINITY;
  int bi = -1;
  for (int c = lane; c < a.ncols; c += 64) {
    float v = p[c];
    for (int s = 1; s < a.splits; ++s) v += p[s * sstride + c];
    if (v > bv) {  // ascending columns per lane: the first of equal values stays
      bv = v;
      bi = c;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    if (a.first) {
      a.best_val[row] = bv;
      a.best_idx[row] = bi < 0 ? -1 : a.col0 + bi;
    } else if (bi >= 0 && (a.best_idx[row] < 0 || bv > a.best_val[row])) {
      a.best_val[row] = bv;
      a.best_idx[row] = a.col0 + bi;
    }
  }
}

// DP start: budget 0 and the reference hold x0; every other budget is empty.
template <class T>
__global__ __launch_bounds__(SEL_THREADS) void init_kernel(InitArgs a) {
  const int q = blockIdx.x;
  const float* x0 = a.x0[q];  // [r][d]
  const int r0 = a.rows[4 * q], rref = a.rows[4 * q + 1], win = a.rows[4 * q + 2];
  const size_t slot = (size_t)a.kmax * a.wmax * a.d;
  const size_t sstride = (size_t)(a.Bm + 1) * slot;
  float* st = a.state + q * sstride;
  const int nslots = a.Bm * a.kmax;  // (budget, beam slot) pairs; slot (0, 0) holds x0
  for (int i = threadIdx.x; i < nslots; i += SEL_THREADS)
    a.valid[(size_t)q * nslots + i] = i == 0 ? 1 : 0;
  for (int i = threadIdx.x; i < nslots * a.mw; i += SEL_THREADS)
    a.masks[(size_t)q * nslots * a.mw + i] = 0;
  __shared__ float scratch[SEL_THREADS / 64];
  const int d4 = a.d / 4;
  for (int t = 0; t < win; ++t) {
    const float* xt = x0 + (size_t)t * a.d;
    float ss[1] = {0.f};
    for (int e4 = threadIdx.x; e4 < d4; e4 += SEL_THREADS) {
      const f32x4 x = *(const f32x4*)(xt + 4 * e4);
      *(f32x4*)(st + (size_t)t * a.d + 4 * e4) = x;
      *(f32x4*)(st + (size_t)a.Bm * slot + (size_t)t * a.d + 4 * e4) = x;
      ss[0] += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    }
    block_sum<1>(ss, scratch);
    const float scale = 1.0f / sqrtf(ss[0] / (float)a.d + a.eps);
    for (int e4 = threadIdx.x; e4 < d4; e4 += SEL_THREADS) {
      const f32x4 x = *(const f32x4*)(xt + 4 * e4);
      if (r0 >= 0) store_act<T>(a.xa, r0 + t, a.d, e4, x, scale);
      if (rref >= 0) store_act<T>(a.xa, rref + t, a.d, e4, x, scale);
    }
  }
}

template <class T>
__global__ __launch_bounds__(SEL_THREADS) void carry_kernel(const float* src, int d, float eps,
                                                           float* state, void* xa) {
  const int t = blockIdx.x;
  const float* x = src + (size_t)t * d;
  __shared__ float scratch[SEL_THREADS / 64];
  const int d4 = d / 4;
  float ss[1] = {0.f};
  for (int e4 = threadIdx.x; e4 < d4; e4 += SEL_THREADS) {
    const f32x4 v = *(const f32x4*)(x + 4 * e4);
    *(f32x4*)(state + (size_t)t * d + 4 * e4) = v;
    ss[0] += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  block_sum<1>(ss, scratch);
  const float scale = 1.0f / sqrtf(ss[0] / (float)d + eps);
  for (int e4 = threadIdx.x; e4 < d4; e4 += SEL_THREADS) {
    const f32x4 v = *(const f32x4*)(x + 4 * e4);
    store_act<T>(xa, t, d, e4, v, scale);
  }
}

template <class T>
__global__ __launch_bounds__(SEL_THREADS) void embed_kernel(const T* w, const int* idx, int d,
                                                           float* out) {
  const int t = blockIdx.x;
  const int tok = idx[t];
  for (int e = threadIdx.x; e < d; e += SEL_THREADS)
    out[(size_t)t * d + e] = tok >= 0 ? to_f32(w[(size_t)tok * d + e]) : 0.f;
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  if (a.splits < 1 || a.splits > GEMM_MAX_SPLITS) return hipErrorInvalidValue;
  const size_t n = (size_t)a.R * (a.d / 4);
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class T>
static void launch_select_t(const SelectArgs& a, hipStream_t s) {
  const dim3 grid(a.n_seqs * (a.B + 1));
  const int it = (a.d / 4 + SELR_THREADS - 1) / SELR_THREADS;
  if (it <= 1)
    hipLaunchKernelGGL((select_reg_kernel<T, 1>), grid, dim3(SELR_THREADS), 0, s, a);
  else if (it <= 2)
    hipLaunchKernelGGL((select_reg_kernel<T, 2>), grid, dim3(SELR_THREADS), 0, s, a);
  else if (it <= SELR_MAXIT)
    hipLaunchKernelGGL((select_reg_kernel<T, SELR_MAXIT>), grid, dim3(SELR_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(select_kernel<T>, grid, dim3(SEL_THREADS), 0, s, a);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.beam > 1) {
    const dim3 grid(a.n_seqs * (a.B + 1));
    if (a.act == ACT_F32)
      hipLaunchKernelGGL(select_beam_kernel<float>, grid, dim3(SELB_THREADS), 0, s, a);
    else
      hipLaunchKernelGGL(select_beam_kernel<bf16>, grid, dim3(SELB_THREADS), 0, s, a);
  } else if (a.rmax > 1) {  // some sequence holds r > 1 token states
    const dim3 grid(a.n_seqs * (a.B + 1));
    if (a.act == ACT_F32)
      hipLaunchKernelGGL(select_win_kernel<float>, grid, dim3(SELW_THREADS), 0, s, a);
    else
      hipLaunchKernelGGL(select_win_kernel<bf16>, grid, dim3(SELW_THREADS), 0, s, a);
  } else if (a.act == ACT_F32) {
    launch_select_t<float>(a, s);
  } else {
    launch_select_t<bf16>(a, s);
  }
  return hipGetLastError();
}

hipError_t launch_lm_argmax(const LmArgmaxArgs& a, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  hipLaunchKernelGGL(lm_argmax_kernel, dim3((a.R + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_init(const InitArgs& a, hipStream_t s) {
  const dim3 grid(a.n_seqs), block(SEL_THREADS);
  if (a.act == ACT_F32)
    hipLaunchKernelGGL(init_kernel<float>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(init_kernel<bf16>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ks

namespace ks {

hipError_t launch_carry(const float* src, int n, int d, float eps, float* state, void* xa,
                        int act, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (act == ACT_F32)
    hipLaunchKernelGGL(carry_kernel<float>, dim3(n), dim3(SEL_THREADS), 0, s, src, d, eps, state, xa);
  else
    hipLaunchKernelGGL(carry_kernel<bf16>, dim3(n), dim3(SEL_THREADS), 0, s, src, d, eps, state, xa);
  return hipGetLastError();
}

hipError_t launch_embed(const void* w_lm, const int* idx, int n, int d, int act, float* out,
                        hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (act == ACT_F32)
    hipLaunchKernelGGL(embed_kernel<float>, dim3(n), dim3(SEL_THREADS), 0, s, (const float*)w_lm,
                       idx, d, out);
  else
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(n), dim3(SEL_THREADS), 0, s, (const bf16*)w_lm,
                       idx, d, out);
  return hipGetLastError();
}

}  // namespace ks
