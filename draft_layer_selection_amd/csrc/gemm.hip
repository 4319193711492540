// Weight-streaming GEMMs of one DP item: all live budget rows of all sequences (plus the
// reference rows) multiply one layer's weight matrix, so every weight byte is read from HBM
// once per item however many budgets are live (the batching of all budgets into one GEMM).
//
// bf16 path (gfx950 MFMA v_mfma_f32_32x32x16_bf16):
//   workgroup = 4 waves, tile = (32*MB rows) x (64 output columns); the 4 waves split each
//   64-wide K step (16 K each), so every weight element is loaded by exactly one lane of one
//   wave straight into registers and every activation element once per tile; the four partial
//   accumulators are summed through LDS in a fixed order (deterministic).  K is split across
//   workgroups only as far as needed to fill the 256 CUs; the consumer adds the splits.
// f32 path: plain LDS-tiled FMA kernel (the small float32 decoder only).
#include "common.h"
#include "kernels.h"

namespace ks {

namespace {

constexpr int RED_PITCH = 64 + 4;

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

template <int MB>
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

  int wrow0, wrow1;
  if (a.mode == GEMM_SWIGLU) {
    wrow0 = nt * 32 + l32;
    wrow1 = a.ff + nt * 32 + l32;
  } else {
    wrow0 = nt * 64 + l32;
    wrow1 = nt * 64 + 32 + l32;
  }
  const int koff = wave * 16 + hi * 8;
  const bf16* W = (const bf16*)a.W;
  const bf16* w0p = W + (size_t)wrow0 * a.K + koff;
  const bf16* w1p = W + (size_t)wrow1 * a.K + koff;
  const bf16* A = (const bf16*)a.A;
  const bf16* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int r = row0 + 32 * mb + l32;
    r = r < a.R ? r : a.R - 1;
    ap[mb] = A + (size_t)r * a.lda + koff;
  }
  const int k0 = sp * a.k_chunk;
  const int k1 = min(a.K, k0 + a.k_chunk);

  f32x16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[mb][0][r] = 0.f;
      acc[mb][1][r] = 0.f;
    }
  }

#pragma unroll 2
  for (int k = k0; k < k1; k += 64) {
    const bf16x8 b0 = *(const bf16x8*)(w0p + k);
    const bf16x8 b1 = *(const bf16x8*)(w1p + k);
    bf16x8 av[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) av[mb] = *(const bf16x8*)(ap[mb] + k);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mb], b0, acc[mb][0], 0, 0, 0);
      acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mb], b1, acc[mb][1], 0, 0, 0);
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
      As[r][c] = (grow < a.R && gk < k1) ? A[(size_t)grow * a.lda + gk] : 0.f;
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

hipError_t launch_gemm(const GemmArgs& a, int act, hipStream_t s) {
  const int total = a.n_tiles * a.m_tiles * a.splits;
  GemmArgs b = a;
  b.per_xcd = (total + 7) / 8;
  const dim3 grid(b.per_xcd * 8), block(256);
  if (act == ACT_F32) {
    hipLaunchKernelGGL(gemm_f32_kernel, grid, block, 0, s, b);
  } else {
    switch (a.mb) {
      case 1: hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, block, 0, s, b); break;
      case 2: hipLaunchKernelGGL(gemm_bf16_kernel<2>, grid, block, 0, s, b); break;
      case 3: hipLaunchKernelGGL(gemm_bf16_kernel<3>, grid, block, 0, s, b); break;
      default: hipLaunchKernelGGL(gemm_bf16_kernel<4>, grid, block, 0, s, b); break;
    }
  }
  return hipGetLastError();
}

}  // namespace ks
