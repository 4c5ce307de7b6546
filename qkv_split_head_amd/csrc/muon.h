// Per-head Newton-Schulz on fused QKV weights: the per-block steps.
//
// DeepSpeed page "[muon] Per-head Newton-Schulz for fused QKV projections",
// "What this PR does": a fused q|k|v weight is a stack of head blocks of
// head_dim rows (in the sectioned and in the interleaved order alike), and the
// update orthogonalises each block on its own, scaled by max(1, rows/cols)**0.5
// of the block.  The iteration is Muon's quintic: on the wide orientation X of a
// block, A = X X^T and X <- a X + (b A + c A^2) X, from X0 = G / (||G||_F + eps).
//
// Every step is X <- P X with P = a I + b A + c A^2, a d x d matrix per block
// (d = the block's short side).  gram_partials_kernel forms A with MFMA from
// X's rows (both operands of X X^T are rows of X, read 16 bytes at a time along
// the long side), as partial sums over column slices; ns_poly_kernel adds the
// partials (gram_reduce_kernel) and forms P, folding in the first step's
// normalisation (||G||_F^2 is the trace of G G^T: A is divided by its square
// and P by the norm) and the last step's scale; the update P X is a plain
// batched GEMM.
#pragma once

#include "device.h"

namespace qkvnr {

constexpr int kNsMaxD = 128;          // largest block side the kernels handle
constexpr int kNsThreads = 256;
constexpr float kNsA = 3.4445f, kNsB = -4.7750f, kNsC = 2.0315f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Partial Gram matrices of bf16 blocks: X [blocks, d, cols] (row stride cols),
// out [blocks, parts, d, d] fp32, out[b][p] = X_b[:, S_p] X_b[:, S_p]^T over the
// column slice S_p = [p * slice, min(cols, (p + 1) * slice)), slice <= 512.
// One workgroup per (block, slice), d / 32 waves.  The workgroup first copies
// its d x slice piece into LDS with coalesced 16-byte loads (all issued before
// any is used), rows padded to 64 chunks of 16 bytes and the chunks of row r
// permuted by c ^ (r mod 16), so that the MFMA operand reads below (16 rows at
// one chunk per pass) fall in 16 different bank groups.  Then wave w forms the
// 32 x 32 tiles of its rows [32 w, 32 w + 32) with v_mfma_f32_32x32x16_bf16:
// lane l's operand is the 8 columns at 8 (l / 32) of each 16-column step of
// row l mod 32 of a 32-row group.  Columns past the slice read as zero.
constexpr int kGramChunks = 64;  // 16-byte chunks per LDS row: 512 columns
template <int D>
__global__ __launch_bounds__(kWave * (D / 32)) void gram_partials_kernel(const uint16_t* __restrict__ x,
                                                                        int64_t cols, int64_t slice,
                                                                        float* __restrict__ out) {
  constexpr int TILES = D / 32, THREADS = kWave * TILES;
  constexpr int PER = D * kGramChunks / THREADS;  // chunks each thread copies (32)
  __shared__ uint4 lds[D * kGramChunks];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int64_t blk = blockIdx.x;
  const int part = blockIdx.y, parts = gridDim.y;
  const int64_t k0 = part * slice;
  const int n8 = static_cast<int>(max<int64_t>(0, min<int64_t>(cols - k0, slice)) / 8);  // chunks of the slice
  const uint16_t* xb = x + blk * D * cols + k0;
  // copy in two halves of PER / 2 loads each (all of a half's loads go out first)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 v[PER / 2];
#pragma unroll
    for (int j = 0; j < PER / 2; ++j) {
      const int i = threadIdx.x + (h * (PER / 2) + j) * THREADS;
      const int r = i / kGramChunks, c = i % kGramChunks;
      v[j] = c < n8 ? ld16(xb + r * cols + c * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < PER / 2; ++j) {
      const int i = threadIdx.x + (h * (PER / 2) + j) * THREADS;
      const int r = i / kGramChunks, c = i % kGramChunks;
      lds[r * kGramChunks + (c ^ (r & 15))] = v[j];
    }
  }
  __syncthreads();
  const int rr = lane % 32, ch = lane / 32;
  f32x16_t acc[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = f32x16_t{};
  const int steps = (n8 + 1) / 2;  // 16-column steps holding data
  for (int s = 0; s < steps; ++s) {
    const int c = 2 * s + ch;
    const int ra = 32 * w + rr;
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, lds[ra * kGramChunks + (c ^ (ra & 15))]);
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int rb = 32 * t + rr;
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, lds[rb * kGramChunks + (c ^ (rb & 15))]);
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
    }
  }
  // C register e of lane l is row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32 of the tile
  float* o = out + (blk * parts + part) * D * D;
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      o[(32 * w + 8 * (e / 4) + 4 * (lane / 32) + e % 4) * D + 32 * t + lane % 32] = acc[t][e];
}

// Sums each block's Gram partials into its partial 0 (in place): one thread
// per element of A, all blocks at once (n = d * d).
__global__ __launch_bounds__(kNsThreads) void gram_reduce_kernel(float* __restrict__ gram, int parts, int n,
                                                                 int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kNsThreads + threadIdx.x;
  if (i >= total) return;
  float* g = gram + (i / n) * parts * n + i % n;
  float s = g[0];
  for (int p = 1; p < parts; ++p) s += g[static_cast<int64_t>(p) * n];
  g[0] = s;
}

// P from the Gram matrix A of each block (held in the block's partial 0, i.e.
// at gram + b * parts * d * d): one workgroup per (block, group of 32 rows of
// P).  The workgroup copies A into LDS and forms its rows of A^2 in 4 x 4
// patches (A is symmetric, so both factors are read along rows of A).
// DT > 0 fixes d at compile time (the common side 128); 0 takes it from `d_rt`.
template <typename OUT, int DT>
__global__ __launch_bounds__(kNsThreads) void ns_poly_kernel(const float* __restrict__ gram, OUT* __restrict__ out,
                                                            int d_rt, int parts, int first, float last_scale,
                                                            float eps) {
  const int d = DT > 0 ? DT : d_rt;
  constexpr int LD = kNsMaxD + 1;  // odd row stride: the column patches of a wave read different banks
  __shared__ float A[kNsMaxD * LD];
  __shared__ float red[kNsThreads / kWave];
  const int64_t blk = blockIdx.x;
  const int row0 = blockIdx.y * 32, rows = min(32, d - row0);
  const float* g = gram + blk * parts * d * d;
  {  // all of the thread's loads first, then the LDS writes (one round trip, not one per element)
    constexpr int CH = kNsMaxD * kNsMaxD / kNsThreads;
    const int n = d * d;
    float v[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = threadIdx.x + j * kNsThreads;
      v[j] = i < n ? g[i] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = threadIdx.x + j * kNsThreads;
      if (i < n) A[(i / d) * LD + i % d] = v[j];
    }
  }
  __syncthreads();
  float inv_n = 1.0f;
  if (first) {  // A = G G^T / (n + eps)^2 and P carries 1 / (n + eps), n = ||G||_F
    float tr = 0.0f;
    for (int i = threadIdx.x; i < d; i += kNsThreads) tr += A[i * LD + i];
    for (int off = kWave / 2; off > 0; off >>= 1) tr += __shfl_xor(tr, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = tr;
    __syncthreads();
    float n2 = 0.0f;
    for (int w = 0; w < kNsThreads / kWave; ++w) n2 += red[w];
    inv_n = 1.0f / (sqrtf(n2) + eps);
  }
  const float a2s = inv_n * inv_n;  // A's normalisation, applied to the products below
  const float s = inv_n * last_scale;
  OUT* o = out + blk * d * d;
  const int pr = (rows + 3) / 4, pc = (d + 3) / 4;
  for (int q = threadIdx.x; q < pr * pc; q += kNsThreads) {
    const int r0 = row0 + (q / pc) * 4, c0 = (q % pc) * 4;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
    for (int k = 0; k < d; ++k) {
      float ar[4], ac[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ar[i] = r0 + i < d ? A[(r0 + i) * LD + k] : 0.0f;
        ac[i] = c0 + i < d ? A[(c0 + i) * LD + k] : 0.0f;  // A[k][c] = A[c][k]
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], ac[j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r0 + i, c = c0 + j;
        if (r < row0 + rows && c < d) {
          // P = a I + b A + c A^2 with A scaled by a2s on the first step
          float p = fmaf(kNsC * a2s * a2s, acc[i][j], kNsB * a2s * A[r * LD + c]);
          if (r == c) p += kNsA;
          p *= s;
          if constexpr (sizeof(OUT) == 2)
            o[r * d + c] = static_cast<OUT>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(p)));
          else
            o[r * d + c] = p;
        }
      }
  }
}

}  // namespace qkvnr
