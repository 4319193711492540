// Weight-streaming GEMMs of one DP item: all live budget rows of all sequences (plus the
// reference rows) multiply one layer's weight matrix, so every weight byte is read from HBM
// once per item however many budgets are live (the batching of all budgets into one GEMM).
//
// bf16 main path (gemm_lds_kernel, gfx950 MFMA v_mfma_f32_32x32x16_bf16):
//   * workgroup = 8 waves = NG column groups (64 output columns each) x (8/NG) K slices;
//     tile = 64*NG columns x 32*MB rows; one workgroup per CU (the LDS ring takes ~128-144 KB);
//   * weights and activations go global -> LDS with global_load_lds_dwordx4 (no registers),
//     8 lanes per 128-byte row segment, in a ring of S stages of 64 K each, so S-1 stages are
//     in flight; the 16-byte slot of chunk c in stage row r is c ^ ((r >> 1) & 7): LDS has
//     64 banks x 4 B and serves 16-byte reads 16 lanes at a time, so 16 consecutive 128-byte
//     rows must land on 16 distinct (row parity, slot) pairs for conflict-free MFMA reads;
//   * the barrier between stages is a bare s_barrier: each wave first waits (vmcnt) for its own
//     loads of the stage, and a fenced barrier would instead drain every load in flight; every
//     wave issues the same number of loads per stage and the tail re-issues the last stage, so
//     the wait count is a compile-time constant and the loop carries no per-stage branches
//     (branchy per-stage bookkeeping cost ~15-20% at large R, measured);
//   * MFMA operands are double-buffered in registers: the LDS reads of the next 16-wide K step
//     alternate with the MFMAs of the current one (order pinned with sched_group_barrier), and
//     the barrier opening the next stage sits after the first MFMAs of a stage's last K step;
//   * activations are re-read from L2 once per column tile, i.e. R/(64*NG) times the weight
//     bytes, so the planner widens the tile (NG=4) when R > 128;
//   * K-slice partial sums are reduced through LDS in a fixed order (deterministic); K is split
//     across workgroups only to fill the 256 CUs, and the consumer adds the splits.
// bf16 K-split projections with 65 .. 256 rows (gemm_areg_kernel): activations straight from L2
//   into MFMA operand registers, weights staged through two LDS buffers, one 256-row tile, so
//   each weight byte is fetched once and the pipeline fill is short (see the kernel's notes).
// bf16 fallback (gemm_bf16_kernel): direct-to-register loads, 64-column tiles, any N % 64 == 0.
// f32 path: plain LDS-tiled FMA kernel (the small float32 decoder only).
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ks {

namespace {

constexpr int RED_PITCH = 64 + 4;

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<0, N>(f);
}

// Sum the four waves' copies of one 32x64 block and write it out (PARTIAL or SWIGLU).
template <class T>
__device__ __forceinline__ void store_block(const GemmArgs& a, float (*red)[32][RED_PITCH],
                                            int row_base, int nt, int sp) {
  const int tid = threadIdx.x;
  if (a.mode == GEMM_PARTIAL) {
    for (int e = tid; e < 32 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      const int grow = row_base + r;
      if (grow >= a.R) continue;
      float v = red[0][r][c];
      v += red[1][r][c];
      v += red[2][r][c];
      v += red[3][r][c];
      a.P[((size_t)sp * a.R + grow) * a.ldp + nt * 64 + c] = v;
    }
  } else {
    T* H = (T*)a.H;
    for (int e = tid; e < 32 * 32; e += 256) {
      const int r = e >> 5, j = e & 31;
      const int grow = row_base + r;
      if (grow >= a.R) continue;
      float g = red[0][r][j];
      g += red[1][r][j];
      g += red[2][r][j];
      g += red[3][r][j];
      float u = red[0][r][32 + j];
      u += red[1][r][32 + j];
      u += red[2][r][32 + j];
      u += red[3][r][32 + j];
      H[(size_t)grow * a.ldh + nt * 32 + j] = from_f32<T>(silu_f(g) * u);
    }
  }
}

// PF = k-steps whose loads are in flight ahead of the MFMAs (register ring buffer): with one
// step in flight a wave waits a full HBM round trip per 64-wide K step.
template <int MB, int PF>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  const int total = a.n_tiles * a.m_tiles * a.splits;
  const int L = xcd_tile(blockIdx.x, a.per_xcd);
  if (L >= total) return;
  const int mt = L % a.m_tiles;
  const int rest = L / a.m_tiles;
  const int sp = rest % a.splits;
  const int nt = rest / a.splits;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int row0 = mt * 32 * MB;
  const int rlim = a.r_live ? min(a.R, *a.r_live) : a.R;
  if (row0 >= rlim) return;

  int wrow0, wrow1;
  if (a.mode == GEMM_SWIGLU) {
    wrow0 = nt * 32 + l32;
    wrow1 = a.ff + nt * 32 + l32;
  } else {
    wrow0 = nt * 64 + l32;
    wrow1 = nt * 64 + 32 + l32;
  }
  const int k0 = sp * a.k_chunk;
  const int k1 = min(a.K, k0 + a.k_chunk);
  const int koff = k0 + wave * 16 + hi * 8;
  const bf16* W = (const bf16*)a.W;
  const bf16* w0p = W + (size_t)wrow0 * a.K + koff;
  const bf16* w1p = W + (size_t)wrow1 * a.K + koff;
  const bf16* A = (const bf16*)a.A;
  const bf16* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int r = row0 + 32 * mb + l32;
    r = r < rlim ? r : rlim - 1;
    if (a.amap) r = a.amap[r];
    ap[mb] = A + (size_t)r * a.lda + koff;
  }
  const int nit = (k1 - k0) / 64;

  f32x16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[mb][0][r] = 0.f;
      acc[mb][1][r] = 0.f;
    }
  }

  bf16x8 wq[PF][2];
  bf16x8 aq[PF][MB];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    if (p < nit) {
      wq[p][0] = *(const bf16x8*)(w0p + p * 64);
      wq[p][1] = *(const bf16x8*)(w1p + p * 64);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) aq[p][mb] = *(const bf16x8*)(ap[mb] + p * 64);
    }
  }
  for (int it = 0; it < nit; it += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (it + p < nit) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[p][mb], wq[p][0], acc[mb][0], 0, 0, 0);
          acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[p][mb], wq[p][1], acc[mb][1], 0, 0, 0);
        }
        const int nx = it + p + PF;
        if (nx < nit) {
          wq[p][0] = *(const bf16x8*)(w0p + nx * 64);
          wq[p][1] = *(const bf16x8*)(w1p + nx * 64);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) aq[p][mb] = *(const bf16x8*)(ap[mb] + nx * 64);
        }
      }
    }
  }

  __shared__ float red[4][32][RED_PITCH];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (row0 + 32 * mb >= a.R) break;  // uniform across the workgroup
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // 32x32 accumulator layout: row = 8*(r/4) + 4*(lane/32) + r%4, col = lane%32
        red[wave][8 * (r >> 2) + 4 * hi + (r & 3)][32 * cb + l32] = acc[mb][cb][r];
      }
    }
    __syncthreads();
    store_block<bf16>(a, red, row0 + 32 * mb, nt, sp);
    __syncthreads();
  }
}

// s_waitcnt with vmcnt = N and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_const() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int NG, int MB, int S>
__global__ __launch_bounds__(512) void gemm_lds_kernel(GemmArgs a) {
  constexpr int KSL = 8 / NG;          // K slices (waves per column group)
  constexpr int KSTEPS = 4 / KSL;      // 16-wide K steps per wave per 64-K stage
  constexpr int WR = 64 * NG;          // weight rows per stage
  constexpr int ROWS = WR + 32 * MB;   // + activation rows
  constexpr int STAGE = ROWS * 128;    // bytes per stage (64 bf16 of K per row)
  constexpr int NCH = ROWS / 8;        // 1 KB chunks (8 rows) per stage
  constexpr int PER_WAVE = (NCH + 7) / 8;
  constexpr int RP = 64 * NG + 4;      // reduction buffer pitch (floats)
  static_assert(KSL * 32 * RP * 4 <= S * STAGE, "reduction buffer must fit in the ring");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S * STAGE];

  const int total = a.n_tiles * a.m_tiles * a.splits;
  const int L = xcd_tile(blockIdx.x, a.per_xcd);
  if (L >= total) return;
  const int mt = L % a.m_tiles;
  const int rest = L / a.m_tiles;
  const int sp = rest % a.splits;
  const int nt = rest / a.splits;
  // wave index as a scalar: the per-wave load counts and waits below become scalar code
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int grp = wave / KSL, ksl = wave % KSL;
  const int row0 = mt * 32 * MB;
  // live-row plan: tiles wholly past the live rows have nothing to compute
  const int rlim = a.r_live ? min(a.R, *a.r_live) : a.R;
  if (row0 >= rlim) return;
  const int k0 = sp * a.k_chunk;
  const int k1 = min(a.K, k0 + a.k_chunk);
  const int nit = (k1 - k0) / 64;
  const bf16* W = (const bf16*)a.W;
  const bf16* A = (const bf16*)a.A;

  // Loader: chunk q = 8 stage rows; lane -> row 8q + lane/8, LDS slot lane%8 which holds the
  // row's global 16-byte chunk (lane%8) ^ ((row >> 1) % 8).
  // Every wave issues PER_WAVE chunks per stage; a wave past the last chunk repeats an earlier
  // chunk into that chunk's own place (same bytes), so the per-stage load count is the same
  // for all waves and the waits below are compile-time constants.
  const bf16* src[PER_WAVE];
  const int rin = lane >> 3;
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    int q = wave + 8 * j;
    q = q < NCH ? q : q - NCH;
    const int r = 8 * q + rin;
    const int cglob = (lane & 7) ^ ((r >> 1) & 7);
    if (r < WR) {
      int wrow;
      if (a.mode == GEMM_SWIGLU)
        wrow = r < WR / 2 ? nt * (WR / 2) + r : a.ff + nt * (WR / 2) + (r - WR / 2);
      else
        wrow = nt * WR + r;
      src[j] = W + (size_t)wrow * a.K + k0 + 8 * cglob;
    } else {
      int ar = row0 + (r - WR);
      ar = ar < rlim ? ar : rlim - 1;
      if (a.amap) ar = a.amap[ar];
      src[j] = A + (size_t)ar * a.lda + k0 + 8 * cglob;
    }
  }
  static_assert(8 * PER_WAVE - NCH <= NCH, "at most one repeat per chunk");
  auto issue = [&](int stage, int slot) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      int q = wave + 8 * j;
      q = q < NCH ? q : q - NCH;
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + stage * 64),
                                       (void*)(smem + slot * STAGE + q * 1024), 16, 0, 0);
    }
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[mb][0][r] = 0.f;
      acc[mb][1][r] = 0.f;
    }
  // Stages past the last one are clamped to it: the repeated loads land in slots that no
  // later stage reads, and every stage issues the same number of loads.
#pragma unroll
  for (int p = 0; p < S - 1; ++p) issue(min(p, nit - 1), p);

  // Software pipeline over the 16-wide K steps: two register buffers of MFMA operands; the
  // operands of the next K step are read from LDS while the MFMAs of the current one run
  // (reads and MFMAs alternate), so the MFMA pipe does not wait for LDS latency.  The barrier
  // that opens stage it+1 is taken inside the last K step of stage it, after its first MFMAs:
  // every operand of stage it is in registers by then, so the refill of its slot is safe, and
  // the MFMAs in flight cover the barrier.  Slot and buffer indices are compile-time constants
  // (the loop is unrolled by U stages), so LDS addresses are immediates and the compiler can
  // tell the DMA targets from the slots being read.
  bf16x8 wf[2][2], af[2][MB];
  auto read_w = [&](auto Jc, auto ksc, auto bc, auto cbc) {
    constexpr int J = decltype(Jc)::value, ks = decltype(ksc)::value;
    constexpr int b = decltype(bc)::value, cb = decltype(cbc)::value;
    const int c = 2 * (ksl * KSTEPS + ks) + hi;
    const int r = 64 * grp + 32 * cb + l32;
    wf[b][cb] = *(const bf16x8*)(smem + J * STAGE + r * 128 + 16 * (c ^ ((r >> 1) & 7)));
  };
  auto read_a = [&](auto Jc, auto ksc, auto bc, auto mbc) {
    constexpr int J = decltype(Jc)::value, ks = decltype(ksc)::value;
    constexpr int b = decltype(bc)::value, mb = decltype(mbc)::value;
    const int c = 2 * (ksl * KSTEPS + ks) + hi;
    const int r = WR + 32 * mb + l32;
    af[b][mb] = *(const bf16x8*)(smem + J * STAGE + r * 128 + 16 * (c ^ ((r >> 1) & 7)));
  };
  // operand read number q (0 .. MB+1) of K step (J, ks) into buffer b, in the order the
  // MFMAs below first use them: W0, A0, W1, A1, A2, ...
  auto read_op = [&](auto Jc, auto ksc, auto bc, auto qc) {
    constexpr int q = decltype(qc)::value;
    if constexpr (q == 0 || q == 2)
      read_w(Jc, ksc, bc, std::integral_constant<int, q / 2>{});
    else
      read_a(Jc, ksc, bc, std::integral_constant<int, q == 1 ? 0 : q - 2>{});
  };
  // MFMA number m (0 .. 2MB-1) of the K step held in buffer b
  auto mfma = [&](auto bc, auto mc) {
    constexpr int b = decltype(bc)::value, m = decltype(mc)::value;
    constexpr int mb = m / 2, cb = m % 2;
    acc[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][mb], wf[b][cb], acc[mb][cb], 0, 0, 0);
  };
  constexpr int NM = 2 * MB, NR = MB + 2;
  // MFMAs first .. NM-1 of buffer b alternating with the NR reads of the next K step, in a
  // scheduling region of its own whose order is pinned (MFMA, LDS read, MFMA, ...): left to
  // itself the scheduler groups the reads after the MFMAs and waits for each group.
  auto interleave = [&](auto bc, auto firstc, auto nJc, auto nksc) {
    constexpr int b = decltype(bc)::value, first = decltype(firstc)::value;
    constexpr int n = NM - first > NR ? NM - first : NR;
    __builtin_amdgcn_sched_barrier(0);
    static_for<n>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (first + i < NM) mfma(bc, std::integral_constant<int, first + i>{});
      if constexpr (i < NR)
        read_op(nJc, nksc, std::integral_constant<int, 1 - b>{}, std::integral_constant<int, i>{});
    });
    static_for<n>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (first + i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int EARLY = 2 * MB - (MB + 2) > 1 ? 2 * MB - (MB + 2) : 1;  // MFMAs before the barrier
  // one stage (slot J, local index Jl within the unrolled group), stage number it
  auto stage = [&](auto Jlc, int it) {
    constexpr int Jl = decltype(Jlc)::value, J = Jl % S, Jn = (Jl + 1) % S;
    static_for<KSTEPS>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      constexpr int b = (Jl * KSTEPS + ks) & 1;
      using B = std::integral_constant<int, b>;
      if constexpr (ks + 1 < KSTEPS) {
        interleave(B{}, std::integral_constant<int, 0>{}, std::integral_constant<int, J>{},
                   std::integral_constant<int, ks + 1>{});
      } else {
        static_for<EARLY>([&](auto mc) { mfma(B{}, mc); });
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_const<(S - 2) * PER_WAVE>();  // this wave's part of stage it+1 landed
        asm volatile("s_barrier" ::: "memory");  // ... and everyone else's; slot J is read out
        issue(min(it + S, nit - 1), J);         // refill it with stage it+S
        __builtin_amdgcn_sched_barrier(0);
        interleave(B{}, std::integral_constant<int, EARLY>{}, std::integral_constant<int, Jn>{},
                   std::integral_constant<int, 0>{});
      }
    });
  };
  // unroll by U stages: a multiple of S (compile-time slots) with an even number of K steps
  // (compile-time buffer parity)
  constexpr int U = (S * KSTEPS) % 2 == 0 ? S : 2 * S;
  wait_vm_const<(S - 2) * PER_WAVE>();  // stage 0
  asm volatile("s_barrier" ::: "memory");
  issue(min(S - 1, nit - 1), S - 1);  // the last slot, unused so far
  static_for<NR>([&](auto qc) {
    read_op(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
            std::integral_constant<int, 0>{}, qc);
  });
  int it0 = 0;
  for (; it0 + U <= nit; it0 += U)
    static_for<U>([&](auto Jlc) { stage(Jlc, it0 + decltype(Jlc)::value); });
  static_for<U>([&](auto Jlc) {
    constexpr int Jl = decltype(Jlc)::value;
    if (it0 + Jl < nit) stage(Jlc, it0 + Jl);
  });
  wait_vm_const<0>();  // repeated tail loads may still be writing the ring the reduction reuses
  __syncthreads();

  float (*red)[32][RP] = (float (*)[32][RP])smem;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (row0 + 32 * mb >= a.R) break;  // uniform across the workgroup
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        red[ksl][8 * (r >> 2) + 4 * hi + (r & 3)][64 * grp + 32 * cb + l32] = acc[mb][cb][r];
    __syncthreads();
    const int tid = threadIdx.x;
    if (a.mode == GEMM_PARTIAL) {
      for (int e = tid; e < 32 * WR; e += 512) {
        const int r = e / WR, cc = e % WR;
        const int grow = row0 + 32 * mb + r;
        if (grow >= a.R) continue;
        float v = red[0][r][cc];
#pragma unroll
        for (int k = 1; k < KSL; ++k) v += red[k][r][cc];
        a.P[((size_t)sp * a.R + grow) * a.ldp + nt * WR + cc] = v;
      }
    } else {
      bf16* H = (bf16*)a.H;
      constexpr int HW = WR / 2;
      for (int e = tid; e < 32 * HW; e += 512) {
        const int r = e / HW, j = e % HW;
        const int grow = row0 + 32 * mb + r;
        if (grow >= a.R) continue;
        float g = red[0][r][j], u = red[0][r][HW + j];
#pragma unroll
        for (int k = 1; k < KSL; ++k) {
          g += red[k][r][j];
          u += red[k][r][HW + j];
        }
        H[(size_t)grow * a.ldh + nt * HW + j] = (bf16)(silu_f(g) * u);
      }
    }
    __syncthreads();
  }
}

// Activations in registers, weights through LDS (rows 65 .. 256 of one item).
//
// Why: in gemm_lds_kernel a stage holds weight and activation rows in one ring, and vector
// loads complete in issue order, so both streams are in flight to the same depth; at 256
// rows an activation stage is twice the 128-column weight stage and only a third of the
// 160 KB ring carries weight bytes (or two 128-row m-tiles fetch each weight line twice).
// Here the activations go straight from L2 into the MFMA operand registers, and LDS holds
// two weight stages only:
//   * workgroup = 8 waves, tile = 128 weight rows (output columns) x 256 activation rows;
//     wave w owns rows 32w .. 32w+31 and all 128 columns (4 accumulator blocks), so every
//     weight byte is fetched from HBM once per item and every activation row once per tile;
//   * K permutation: in 16-wide step ks of a 64-K stage, lane half hi supplies K elements
//     32hi + 8ks .. +7 for both operands (the MFMA sums over whichever K it is given, as
//     long as both operands agree), so a lane's activations for a stage are 64 contiguous
//     bytes: four 16-byte loads, D stages ahead of their use, in D+1 register sets;
//   * weights: every wave loads 2 of the stage's 16 1 KB chunks into registers D stages
//     ahead (D register sets) and stores them to the LDS stage buffer one stage before use;
//     the stage buffers alternate, and the barrier opening stage t (after each wave's LDS
//     stores have completed) both publishes stage t and frees the buffer stage t+1 goes to;
//   * only ordinary vector loads are in flight, which complete in issue order, so the
//     compiler's waits before each use are exact (LDS-DMA loads mixed with register loads
//     make it drain the whole queue before every use of a loaded register);
//   * the loop is unrolled so register sets and stage buffers are compile-time constants;
//   * epilogue straight from the accumulators: the K-split partial sums of each split
//     (XCD-local split order); the SwiGLU GEMM stays on gemm_lds_kernel (not faster here).
// Rows past the live count (r_live) are skipped a wave at a time: such a wave only helps to
// stage the weights.
constexpr int AREG_ROWS = 256;  // activation rows per tile
constexpr int AREG_COLS = 128;  // weight rows (output columns) per tile
constexpr int AREG_MIN_ROWS = 64;     // at or below: gemm_lds_kernel (deeper weight ring)
constexpr int AREG_DEFAULT_DEPTH = 3;  // measured: depth 4 no faster, 5 spills registers

template <int A, int B>
struct Lcm {
  static constexpr int gcd(int x, int y) { return y == 0 ? x : gcd(y, x % y); }
  static constexpr int value = A / gcd(A, B) * B;
};

// Weight stage buffer I of the register-activation kernel: one LDS object per buffer, so the
// compiler's alias analysis tells the buffer being stored from the one being read.
template <int I>
__device__ __forceinline__ unsigned char* areg_slot() {
  __shared__ __attribute__((aligned(1024))) unsigned char buf[AREG_COLS * 128];
  return buf;
}

template <int D>
__global__ __launch_bounds__(512) void gemm_areg_kernel(GemmArgs a) {
  constexpr int NAB = D + 1;  // activation register sets
  constexpr int NWB = D;      // weight register sets
  constexpr int U = Lcm<Lcm<NAB, NWB>::value, 2>::value;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

  const int total = a.n_tiles * a.splits;
  const int L = xcd_tile(blockIdx.x, a.per_xcd);
  if (L >= total) return;
  const int sp = L / a.n_tiles;  // consecutive tiles (one XCD) share a K split
  const int nt = L % a.n_tiles;
  const int rlim = a.r_live ? min(a.R, *a.r_live) : a.R;
  if (rlim <= 0) return;  // uniform across the workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool active = wave * 32 < rlim;  // wave-uniform
  const int k0 = sp * a.k_chunk;
  const int k1 = min(a.K, k0 + a.k_chunk);
  const int nit = (k1 - k0) / 64;
  if (nit <= 0) return;  // the planner never makes an empty split
  const int last = nit - 1;
  const bf16* W = (const bf16*)a.W;
  const bf16* Ap = (const bf16*)a.A;

  // weight chunks of this wave: q = w and w + 8 (8 stage rows each); lane -> row
  // 8q + lane/8, 16-byte slot lane%8 of the row <- its global chunk (lane%8) ^ ((row>>1)%8),
  // which keeps the operand reads below conflict-free
  const bf16* wsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * (wave + 8 * j) + (lane >> 3);
    const int cglob = (lane & 7) ^ ((r >> 1) & 7);
    wsrc[j] = W + (size_t)(nt * AREG_COLS + r) * a.K + k0 + 8 * cglob;
  }
  // activations of this lane's row: K elements 32hi .. 32hi+31 of each stage
  int arow = wave * 32 + l32;
  arow = arow < rlim ? arow : rlim - 1;
  if (a.amap) arow = a.amap[arow];
  const bf16* asrc = Ap + (size_t)arow * a.lda + k0 + 32 * hi;

  bf16x8 av[NAB][4];
  u32x4 wv[NWB][2];
  auto load_a = [&](auto bc, int stage) {
    constexpr int b = decltype(bc)::value;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) av[b][ks] = *(const bf16x8*)(asrc + stage * 64 + 8 * ks);
  };
  auto load_w = [&](auto bc, int stage) {
    constexpr int b = decltype(bc)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j) wv[b][j] = *(const u32x4*)(wsrc[j] + stage * 64);
  };
  auto store_w = [&](auto bc, auto sc) {
    constexpr int b = decltype(bc)::value, sl = decltype(sc)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *(u32x4*)(areg_slot<sl>() + (wave + 8 * j) * 1024 + lane * 16) = wv[b][j];
  };

  f32x16 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  // operand read offset of K step ks: stage row 32cb + l32 (block cb adds 4 KB), chunk
  // 4hi + ks; the swizzle (row >> 1) % 8 does not depend on cb
  int woff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) woff[ks] = l32 * 128 + 16 * ((4 * hi + ks) ^ ((l32 >> 1) & 7));

  // C = whether this wave computes (instantiated once per case: straight-line code between
  // the barriers)
  auto run = [&](auto cc) {
    constexpr bool C = decltype(cc)::value;
    // prologue: weights 0 .. D-1 and activations 0 .. D in flight, weights 0 stored
    static_for<NWB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      load_w(ic, min(i, last));
      if constexpr (C) load_a(ic, min(i, last));
    });
    if constexpr (C) load_a(std::integral_constant<int, D>{}, min(D, last));
    store_w(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    load_w(std::integral_constant<int, 0>{}, min(NWB, last));

    // stage t (j = t % U): wait for this wave's LDS stores, barrier (stage t published,
    // stage t-1 read out), MFMAs of stage t, store weights t+1 and load weights t+1+D into
    // their register set, load activations t+D+1 into the set stage t used
    auto stage = [&](auto jc, int t) {
      constexpr int j = decltype(jc)::value;
      constexpr int sl = j % 2, b = j % NAB, bw = (j + 1) % NWB;
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
      if constexpr (C) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 wop[4];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            wop[cb] = *(const bf16x8*)(areg_slot<sl>() + cb * 4096 + woff[ks]);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[b][ks], wop[cb], acc[cb], 0, 0, 0);
        }
      }
      store_w(std::integral_constant<int, bw>{}, std::integral_constant<int, (j + 1) % 2>{});
      load_w(std::integral_constant<int, bw>{}, min(t + 1 + NWB, last));
      if constexpr (C) load_a(std::integral_constant<int, b>{}, min(t + NAB, last));
    };
    int t0 = 0;
    for (; t0 + U <= nit; t0 += U)
      static_for<U>([&](auto jc) { stage(jc, t0 + decltype(jc)::value); });
    static_for<U>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if (t0 + j < nit) stage(jc, t0 + j);
    });
    // loads past the last stage (clamped) may still be writing registers
    __builtin_amdgcn_s_waitcnt(0);
  };
  if (active)
    run(std::true_type{});
  else
    run(std::false_type{});
  if (!active) return;

  // accumulator layout: block cb, register r -> row 32w + 8(r/4) + 4hi + r%4, column
  // 32cb + l32 of the tile
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int grow = wave * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (grow >= a.R) continue;
    float* prow = a.P + ((size_t)sp * a.R + grow) * a.ldp + nt * AREG_COLS + l32;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) prow[32 * cb] = acc[cb][r];
  }
}

// float32 path: tile 32 rows x 64 columns, K staged through LDS 32 at a time; thread
// (ty, tx) owns rows {ty, ty+16} and columns tx*4..tx*4+3.
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  const int total = a.n_tiles * a.m_tiles * a.splits;
  const int L = xcd_tile(blockIdx.x, a.per_xcd);
  if (L >= total) return;
  const int mt = L % a.m_tiles;
  const int rest = L / a.m_tiles;
  const int sp = rest % a.splits;
  const int nt = rest / a.splits;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const int row0 = mt * 32;
  if (a.r_live && row0 >= min(a.R, *a.r_live)) return;
  const float* A = (const float*)a.A;
  const float* W = (const float*)a.W;

  __shared__ float As[32][33];
  __shared__ float Ws[64][33];
  __shared__ float red[1][32][RED_PITCH];

  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const int k0 = sp * a.k_chunk;
  const int k1 = min(a.K, k0 + a.k_chunk);
  for (int kk = k0; kk < k1; kk += 32) {
    for (int e = tid; e < 32 * 32; e += 256) {
      const int r = e >> 5, c = e & 31;
      const int grow = row0 + r, gk = kk + c;
      const int arow = (a.amap && grow < a.R) ? a.amap[grow] : grow;
      As[r][c] = (grow < a.R && gk < k1) ? A[(size_t)arow * a.lda + gk] : 0.f;
    }
    for (int e = tid; e < 64 * 32; e += 256) {
      const int n = e >> 5, c = e & 31;
      int wrow;
      if (a.mode == GEMM_SWIGLU)
        wrow = n < 32 ? nt * 32 + n : a.ff + nt * 32 + (n - 32);
      else
        wrow = nt * 64 + n;
      const int gk = kk + c;
      Ws[n][c] = (wrow < (a.mode == GEMM_SWIGLU ? 2 * a.ff : a.N) && gk < k1)
                     ? W[(size_t)wrow * a.K + gk]
                     : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < 32; ++c) {
      const float a0 = As[ty][c], a1 = As[ty + 16][c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float wv = Ws[tx * 4 + j][c];
        acc[0][j] = fmaf(a0, wv, acc[0][j]);
        acc[1][j] = fmaf(a1, wv, acc[1][j]);
      }
    }
    __syncthreads();
  }
  // reuse the 4-way reduction layout with three zero copies so both paths share the epilogue
  for (int j = 0; j < 4; ++j) {
    red[0][ty][tx * 4 + j] = acc[0][j];
    red[0][ty + 16][tx * 4 + j] = acc[1][j];
  }
  __syncthreads();
  if (a.mode == GEMM_PARTIAL) {
    for (int e = tid; e < 32 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      const int grow = row0 + r;
      if (grow >= a.R || nt * 64 + c >= a.N) continue;
      a.P[((size_t)sp * a.R + grow) * a.ldp + nt * 64 + c] = red[0][r][c];
    }
  } else {
    float* H = (float*)a.H;
    for (int e = tid; e < 32 * 32; e += 256) {
      const int r = e >> 5, j = e & 31;
      const int grow = row0 + r;
      if (grow >= a.R || nt * 32 + j >= a.ff) continue;
      H[(size_t)grow * a.ldh + nt * 32 + j] = silu_f(red[0][r][j]) * red[0][r][32 + j];
    }
  }
}

}  // namespace

// Activation stages in flight of the activations-in-registers GEMM (0 = not used); the
// KNAPSPEC_GEMM_AREG environment variable (0, 3 or 4) overrides the default, read once.
int areg_depth() {
  static const int depth = [] {
    const char* e = std::getenv("KNAPSPEC_GEMM_AREG");
    if (!e || !*e) return AREG_DEFAULT_DEPTH;
    const int v = std::atoi(e);
    return (v == 3 || v == 4) ? v : 0;
  }();
  return depth;
}

GemmPlan plan_gemm(int act, int R, int N, int K, int mode, int ff, size_t cap_floats) {
  GemmPlan p{};
  const int ncols = mode == GEMM_SWIGLU ? 2 * ff : N;
  const int kstep = act == ACT_F32 ? 32 : 64;
  const int kiters = (K + kstep - 1) / kstep;
  auto finish = [&](int s) {
    const int per = (kiters + s - 1) / s;
    p.k_chunk = per * kstep;
    p.splits = (kiters + per - 1) / per;
  };
  if (act == ACT_F32) {
    p.ng = 0;
    p.mb = 1;
    p.m_tiles = (R + 31) / 32;
    p.n_tiles = mode == GEMM_SWIGLU ? (ff + 31) / 32 : (N + 63) / 64;
    int s = 1;
    if (mode != GEMM_SWIGLU) {
      s = std::max(1, 512 / std::max(1, p.n_tiles * p.m_tiles));
      s = std::min(std::min(s, GEMM_MAX_SPLITS), std::max(1, kiters / 4));
      while (s > 1 && (size_t)s * R * N > cap_floats) --s;
    }
    finish(s);
    return p;
  }
  const bool k_ok = K % 64 == 0;
  const int areg = areg_depth();
  if (areg > 0 && mode == GEMM_PARTIAL && k_ok && R > AREG_MIN_ROWS && R <= AREG_ROWS &&
      N % AREG_COLS == 0) {
    // activations-in-registers kernel (K-split projections only: on the SwiGLU GEMM it
    // measured no faster than gemm_lds_kernel): one m-tile; K splits fill the 256 CUs, each
    // split at least 2*(areg+1) stages long so the pipeline fill stays small
    p.areg = areg;
    p.ng = 0;
    p.mb = AREG_ROWS / 32;
    p.m_tiles = 1;
    p.n_tiles = N / AREG_COLS;
    int s = std::max(1, 256 / p.n_tiles);
    s = std::min(s, GEMM_MAX_SPLITS);
    s = std::max(1, std::min(s, kiters / (2 * (areg + 1))));
    while (s > 1 && (size_t)s * R * N > cap_floats) --s;
    finish(s);
    return p;
  }
  if (mode == GEMM_PARTIAL && k_ok && N % 128 == 0) {
    // K-split LDS kernel: pick the tile (64*ng columns x 32*mb rows) and split count with the
    // least modelled time: rounds of 256 workgroups x bytes each workgroup stages through LDS
    // (its K stages plus 2 stages' worth of start-up), plus the fp32 partial sums written and
    // read back (weighted 0.01 per byte).  The split count is capped at K/(4R), which keeps the
    // partial traffic within 2x the weight bytes where the rows are many; 256-column tiles
    // only above 128 rows.  Fitted to cold-weight timings of the Llama-3-8B shapes (q|k|v, O
    // and down projections, R = 32 .. 245, GEMM plus split reduction): within 2% of the best
    // tile and split count per shape, against 5% for a fixed 256-workgroup target.
    const int smax = std::max(1, std::min(GEMM_MAX_SPLITS, K / std::max(1, 4 * R)));
    double best = -1;
    for (int ng : {2, 4}) {
      if (ng == 4 && (N % 256 != 0 || R <= 128)) continue;
      for (int mb = 1; mb <= 4; ++mb) {
        const int mt = (R + 32 * mb - 1) / (32 * mb), nt = N / (64 * ng), tiles = mt * nt;
        int s = std::min(smax, tiles < 256 ? 256 / tiles : 1);
        s = std::max(1, std::min(s, std::max(1, kiters / 4)));
        while (s > 1 && (size_t)s * R * N > cap_floats) --s;
        const int per = (kiters + s - 1) / s;
        s = (kiters + per - 1) / per;
        const double rounds = (double)((mt * nt * s + 255) / 256);
        const double t = rounds * (64.0 * ng + 32.0 * mb) * 128.0 * (per + 2) +
                         0.01 * (double)s * R * N * 8.0;
        if (best < 0 || t < best) {
          best = t;
          p.ng = ng;
          p.mb = mb;
          p.m_tiles = mt;
          p.n_tiles = nt;
          p.k_chunk = per * 64;
          p.splits = s;
        }
      }
    }
    return p;
  }
  p.m_tiles = (R + 127) / 128;
  p.mb = (R + 32 * p.m_tiles - 1) / (32 * p.m_tiles);
  if (k_ok && R > 128 && ncols % 256 == 0 && (mode != GEMM_SWIGLU || ff % 128 == 0))
    p.ng = 4;
  else if (k_ok && ncols % 128 == 0 && (mode != GEMM_SWIGLU || ff % 64 == 0))
    p.ng = 2;
  else
    p.ng = 0;
  const int cols = p.ng ? 64 * p.ng : 64;
  p.n_tiles = mode == GEMM_SWIGLU ? ff / (cols / 2) : N / cols;
  int s = 1;
  if (mode != GEMM_SWIGLU) {
    // direct-load fallback kernel (N not a multiple of 128 or K of 64)
    const int tiles = p.n_tiles * p.m_tiles;
    s = std::max(1, 512 / std::max(1, tiles));
    s = std::min(std::min(s, GEMM_MAX_SPLITS), std::max(1, kiters / 4));
    while (s > 1 && (size_t)s * R * N > cap_floats) --s;
  }
  finish(s);
  return p;
}

hipError_t launch_gemm(const GemmArgs& a, int act, hipStream_t s) {
  const int total = a.n_tiles * a.m_tiles * a.splits;
  GemmArgs b = a;
  b.per_xcd = (total + 7) / 8;
  const dim3 grid(b.per_xcd * 8);
  if (act == ACT_F32) {
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, b);
  } else if (a.areg > 0) {
    if (a.m_tiles != 1 || a.R > AREG_ROWS || a.mode != GEMM_PARTIAL) return hipErrorInvalidValue;
    switch (a.areg) {
      case 3: hipLaunchKernelGGL((gemm_areg_kernel<3>), grid, dim3(512), 0, s, b); break;
      case 4: hipLaunchKernelGGL((gemm_areg_kernel<4>), grid, dim3(512), 0, s, b); break;
      default: return hipErrorInvalidValue;
    }
  } else if (a.ng == 4) {
    switch (a.mb) {
      case 1: hipLaunchKernelGGL((gemm_lds_kernel<4, 1, 4>), grid, dim3(512), 0, s, b); break;
      case 2: hipLaunchKernelGGL((gemm_lds_kernel<4, 2, 3>), grid, dim3(512), 0, s, b); break;
      case 3: hipLaunchKernelGGL((gemm_lds_kernel<4, 3, 3>), grid, dim3(512), 0, s, b); break;
      default: hipLaunchKernelGGL((gemm_lds_kernel<4, 4, 3>), grid, dim3(512), 0, s, b); break;
    }
  } else if (a.ng == 2) {
    switch (a.mb) {
      case 1: hipLaunchKernelGGL((gemm_lds_kernel<2, 1, 7>), grid, dim3(512), 0, s, b); break;
      case 2: hipLaunchKernelGGL((gemm_lds_kernel<2, 2, 6>), grid, dim3(512), 0, s, b); break;
      case 3: hipLaunchKernelGGL((gemm_lds_kernel<2, 3, 5>), grid, dim3(512), 0, s, b); break;
      default: hipLaunchKernelGGL((gemm_lds_kernel<2, 4, 4>), grid, dim3(512), 0, s, b); break;
    }
  } else {
    switch (a.mb) {
      case 1: hipLaunchKernelGGL((gemm_bf16_kernel<1, 8>), grid, dim3(256), 0, s, b); break;
      case 2: hipLaunchKernelGGL((gemm_bf16_kernel<2, 6>), grid, dim3(256), 0, s, b); break;
      case 3: hipLaunchKernelGGL((gemm_bf16_kernel<3, 5>), grid, dim3(256), 0, s, b); break;
      default: hipLaunchKernelGGL((gemm_bf16_kernel<4, 4>), grid, dim3(256), 0, s, b); break;
    }
  }
  return hipGetLastError();
}

}  // namespace ks
