// Live-row plan of a DP item, built on the device between the previous item's select and the
// item's first GEMM, so that cells pruned by tau or the skip cap (the review's Figure 4:
// pruning the DP's candidate states cuts its memory and optimisation work) also leave the
// item's GEMM rows, attention query blocks and partial results.
//
// One workgroup of 1024 threads:
//   1. a prefix count over each sequence's live candidate sources (valid flag set and
//      b + w_i <= B - 1) gives each live source its row -- block-wide with one budget per
//      thread for a single sequence, else one wave per sequence (16 at a time); the maps of
//      the item (activation row, sequence, window token, state slot, execute row of the target
//      budget) are rewritten, the reference follows the sequence's live sources;
//   2. attention items: each sequence's context split count for its live rows, by the cost
//      model of the host planner (fewest dispatch rounds x (tiles per workgroup + fixed cost),
//      ties to fewer workgroups, then to the earlier candidate), every candidate evaluated by a
//      thread of its own and the minimum taken over the block;
//   3. the layer's work list: (sequence, KV head, split) groups of query blocks dealt to the
//      8 dies round-robin (list position p runs on die p % 8), the query blocks of a group
//      consecutive on its die so the die's L2 serves their shared K/V reads.
#include "common.h"
#include "kernels.h"

namespace ks {

namespace {

constexpr int CW = COMPACT_THREADS / 64;  // waves

// Barrier for LDS traffic only: the kernel's global stores are never read back by it, so the
// barrier does not wait for them (a full __syncthreads waits for every store in flight).
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Exclusive prefix sum of v over the workgroup (thread order); *total = sum of all v.
__device__ int block_excl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  lds_sync();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < CW; ++w) {
    const int s = s_wave[w];
    base += w < wave ? s : 0;
    tot += s;
  }
  *total = tot;
  return base + x - v;
}

__device__ unsigned long long block_min_u64(unsigned long long v, unsigned long long* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)v, o, 64);
    const unsigned hi = __shfl_xor((unsigned)(v >> 32), o, 64);
    const unsigned long long y = ((unsigned long long)hi << 32) | lo;
    v = y < v ? y : v;
  }
  if (lane == 0) s_wave[wave] = v;
  lds_sync();
  unsigned long long m = s_wave[0];
#pragma unroll
  for (int w = 1; w < CW; ++w) m = s_wave[w] < m ? s_wave[w] : m;
  return m;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// exclusive prefix sum of v over the wave's lanes
__device__ __forceinline__ int wave_excl_scan(int v) {
  const int lane = threadIdx.x & 63;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x - v;
}

// number of i in [0, n) with i % 8 == x
__device__ __forceinline__ int count_mod8(int n, int x) { return n > x ? (n - x + 7) / 8 : 0; }

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(COMPACT_THREADS) void compact_kernel(CompactArgs a) {
  __shared__ int s_wave[CW];
  __shared__ unsigned long long s_wmin[CW];
  __shared__ int s_M[COMPACT_MAX_SEQS], s_off[COMPACT_MAX_SEQS];
  __shared__ int s_qb[COMPACT_MAX_SEQS], s_tiles[COMPACT_MAX_SEQS], s_ns[COMPACT_MAX_SEQS];
  __shared__ int s_gp[COMPACT_MAX_SEQS + 1];
  __shared__ int s_load[8];
  __shared__ int s_R;
  const int tid = threadIdx.x;
  const int S = a.n_seqs;
  // the layer's context lengths, loaded with the first sequence's inputs
  const int ctx_t = (a.aseq && tid < S) ? a.aseq[tid].ctx : 0;

  // ---- 1. rows.  One wave per sequence (sequences in parallel); lane l holds the contiguous
  //      budgets [l*per, (l+1)*per), so a wave-wide exclusive prefix of the lanes' live counts
  //      plus the count within the lane is a source's rank in budget order.
  const int wave = tid >> 6, lane = tid & 63;
  if (S == 1) {
    // one sequence: thread b holds budget b, a block-wide prefix count gives the ranks
    const int w = a.info[0].w, wr = a.info[0].win;
    const int next_ref = a.prev_info[0].next_ref_row;
    const int b = tid;
    const bool inb = b < a.B;  // loads independent of w, issued together
    const int vflag = inb ? a.valid[(size_t)b * a.kmax] : 0;
    const int prow = inb ? a.prev_next_row[(size_t)b * a.kmax] : 0;
    const bool cand = inb && b + w <= a.B - 1;
    const bool live = cand && vflag != 0;
    int nlive;
    const int rank = block_excl_scan(live ? 1 : 0, s_wave, &nlive);
    if (cand) {
      const int row = rank * wr;
      a.exec_row[(size_t)(b + w) * a.kmax] = live ? row : -1;
      if (live)
        for (int t = 0; t < wr; ++t) {
          a.amap[row + t] = prow + t;
          a.row_seq[row + t] = 0;
          a.row_tok[row + t] = t;
          a.row_state[row + t] = (int)((size_t)b * a.kmax * a.wmax + t);
        }
    }
    const int ref = nlive * wr;
    if (tid < wr) {
      a.amap[ref + tid] = next_ref + tid;
      a.row_seq[ref + tid] = 0;
      a.row_tok[ref + tid] = tid;
      a.row_state[ref + tid] = (int)((size_t)a.Bm * a.kmax * a.wmax + tid);
    }
    if (tid == 0) {
      a.info[0].row_off = 0;
      a.info[0].M = (nlive + 1) * wr;
      a.info[0].ref_row = ref;
      s_M[0] = (nlive + 1) * wr;
      s_off[0] = 0;
      s_R = (nlive + 1) * wr;
    }
    lds_sync();
  } else {
    // several sequences: one wave per sequence; lane l holds the contiguous budgets
    // [l*per, (l+1)*per), so a wave-wide exclusive prefix of the lanes' live counts plus the
    // count within the lane is a source's rank in budget order
    const int per = (a.B + 63) / 64;
    for (int q = wave; q < S; q += CW) {  // pass A: live sources of each sequence
      const int w = a.info[q].w, wr = a.info[q].win;
      int n = 0;
      for (int k = 0; k < per; ++k) {
        const int b = lane * per + k;
        if (b < a.B && b + w <= a.B - 1 && a.valid[((size_t)q * a.Bm + b) * a.kmax]) ++n;
      }
      const int total = wave_sum(n);
      if (lane == 0) s_M[q] = (total + 1) * wr;
    }
    lds_sync();
    if (tid == 0) {
      int r = 0;
      for (int q = 0; q < S; ++q) {
        s_off[q] = r;
        r += s_M[q];
      }
      s_R = r;
    }
    lds_sync();
    for (int q = wave; q < S; q += CW) {  // pass B: maps
      const int w = a.info[q].w, wr = a.info[q].win;
      const int next_ref = a.prev_info[q].next_ref_row;
      const int row_off = s_off[q];
      const size_t st_q = (size_t)q * (a.Bm + 1) * a.kmax;  // first state slot of the sequence
      int n = 0;
      for (int k = 0; k < per; ++k) {
        const int b = lane * per + k;
        if (b < a.B && b + w <= a.B - 1 && a.valid[((size_t)q * a.Bm + b) * a.kmax]) ++n;
      }
      int rank = wave_excl_scan(n);
      for (int k = 0; k < per; ++k) {
        const int b = lane * per + k;
        if (!(b < a.B && b + w <= a.B - 1)) continue;
        const size_t qb = (size_t)q * a.Bm + b;
        const bool live = a.valid[qb * a.kmax] != 0;
        const int row = row_off + rank * wr;
        a.exec_row[(qb + w) * a.kmax] = live ? row : -1;
        if (!live) continue;
        const int prow = a.prev_next_row[qb * a.kmax];
        for (int t = 0; t < wr; ++t) {
          a.amap[row + t] = prow + t;
          a.row_seq[row + t] = q;
          a.row_tok[row + t] = t;
          a.row_state[row + t] = (int)((st_q + (size_t)b * a.kmax) * a.wmax + t);
        }
        ++rank;
      }
      const int ref = row_off + s_M[q] - wr;
      if (lane < wr) {
        a.amap[ref + lane] = next_ref + lane;
        a.row_seq[ref + lane] = q;
        a.row_tok[ref + lane] = lane;
        a.row_state[ref + lane] = (int)((st_q + (size_t)a.Bm * a.kmax) * a.wmax + lane);
      }
      if (lane == 0) {
        a.info[q].row_off = row_off;
        a.info[q].M = s_M[q];
        a.info[q].ref_row = ref;
      }
    }
  }
  const int R = s_R;
  for (int c = R + tid; c < a.R_plan; c += COMPACT_THREADS) {
    a.amap[c] = 0;
    a.row_seq[c] = 0;
    a.row_tok[c] = 0;
    a.row_state[c] = 0;
  }
  if (tid == 0) *a.r_live = R;
  if (!a.aseq) return;

  // ---- 2. context splits of the live rows
  const int G = a.hq / a.hkv;
  if (tid < S) {
    s_qb[tid] = ceil_div(G * s_M[tid], a.qb_rows);
    s_tiles[tid] = ceil_div(ctx_t, 64);
  }
  lds_sync();
  int xmin = 1, tmax = 0, qbsum = 0;
  for (int q = 0; q < S; ++q) {
    qbsum += s_qb[q];
    if (s_tiles[q] <= 0) continue;
    xmin = max(xmin, ceil_div(s_tiles[q], a.max_split));
    tmax = max(tmax, s_tiles[q]);
  }
  // Dealt round-robin, a sequence's n groups give each die floor(n/8) or ceil(n/8) of them,
  // so a die holds at most count/8 + sum_q qblocks_q entries: the list ends before
  // count + pad.
  const long long pad = 8LL * (qbsum + 1);
  unsigned long long best = ~0ull;
  const int ncand = 1 + S * a.max_split;
  for (int ci = tid; ci < ncand && tmax > 0; ci += COMPACT_THREADS) {
    int x = tmax;
    if (ci > 0) {
      const int q = (ci - 1) / a.max_split, k = (ci - 1) % a.max_split + 1;
      if (s_tiles[q] <= 0) continue;
      x = ceil_div(s_tiles[q], k);
    }
    if (x < xmin || x > tmax) continue;
    long long count = 0, parts = 0;
    for (int q = 0; q < S; ++q) {
      if (s_tiles[q] <= 0) continue;
      const int ns = ceil_div(s_tiles[q], x);
      count += (long long)a.hkv * s_qb[q] * ns;
      parts += (long long)s_M[q] * a.hq * ns;
    }
    if (x != tmax && (parts > a.part_cap || count + pad > a.work_cap)) continue;
    const long long cost = (count + a.slots - 1) / a.slots * (x + 4);
    if (cost >= (1LL << 24) || count >= (1LL << 28)) continue;  // outside the key's fields
    const unsigned long long key = ((unsigned long long)cost << 40) |
                                   ((unsigned long long)count << 12) | (unsigned long long)ci;
    best = key < best ? key : best;
  }
  best = block_min_u64(best, s_wmin);
  int X = tmax;
  if (tmax > 0 && best != ~0ull) {
    const int ci = (int)(best & 4095);
    if (ci > 0) X = ceil_div(s_tiles[(ci - 1) / a.max_split], (ci - 1) % a.max_split + 1);
  }
  int nsplit = 0;
  if (tid < S) {
    const int q = tid;
    const int ns = (s_tiles[q] > 0 && X > 0) ? ceil_div(s_tiles[q], X) : 0;
    const int chunk = ns > 0 ? ceil_div(s_tiles[q], ns) * 64 : 64;
    nsplit = ctx_t > 0 ? ceil_div(ctx_t, chunk) : 0;
    s_ns[q] = nsplit;
    AttnSeq* as = a.aseq + q;
    as->row_off = s_off[q];
    as->M = s_M[q];
    as->nsplit = nsplit;
    as->chunk = chunk;
    // the smallest multiple of 32 whose s_qb[q] blocks cover the KV head's G*M query rows
    const int per = s_qb[q] > 0 ? ceil_div(G * s_M[q], s_qb[q]) : 0;
    as->qrows = (per + 31) / 32 * 32;
  }
  lds_sync();  // s_ns
  if (tid == 0) {
    long long part = 0;
    int gp = 0;
    for (int q = 0; q < S; ++q) {
      a.aseq[q].part_off = (int)part;
      part += (long long)s_ns[q] * s_M[q] * a.hq;
      s_gp[q] = gp;
      gp += a.hkv * s_ns[q];
    }
    s_gp[S] = gp;
  }
  lds_sync();  // s_gp
  if (tid < 8) {  // entries dealt to die x
    int ld = 0;
    for (int q = 0; q < S; ++q)
      ld += s_qb[q] * (count_mod8(s_gp[q + 1], tid) - count_mod8(s_gp[q], tid));
    s_load[tid] = ld;
  }
  lds_sync();  // s_load

  // ---- 3. work list: positions past a die's entries are empty, the rest hold the groups
  for (int p = tid; p < a.work_cap; p += COMPACT_THREADS)
    if ((p >> 3) >= s_load[p & 7]) a.work[p] = make_int4(-1, 0, 0, 0);
  const int ngroups = s_gp[S];
  for (int g = tid; g < ngroups; g += COMPACT_THREADS) {
    int q = 0;
    while (q + 1 < S && s_gp[q + 1] <= g) ++q;
    const int local = g - s_gp[q];
    const int c = local / s_ns[q], sp = local % s_ns[q];
    const int x = g & 7;
    // entries of die x before this group: the query blocks of the earlier groups dealt to it
    int off = 0;
    for (int q2 = 0; q2 < q; ++q2)
      off += s_qb[q2] * (count_mod8(s_gp[q2 + 1], x) - count_mod8(s_gp[q2], x));
    off += s_qb[q] * (count_mod8(g, x) - count_mod8(s_gp[q], x));
    for (int k = 0; k < s_qb[q]; ++k) {
      const long long p = (long long)(off + k) * 8 + x;
      if (p < a.work_cap) a.work[p] = make_int4(q, c, k, sp);
    }
  }
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  if (a.n_seqs < 1 || a.n_seqs > COMPACT_MAX_SEQS || a.B > COMPACT_THREADS)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(COMPACT_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace ks
