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
// partials as it loads them and forms P, folding in the first step's
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
// column slice S_p = [p * slice, min(cols, (p + 1) * slice)).
// One workgroup per (block, slice), d / 32 waves, streams the block's d rows
// through LDS in chunks of 64 columns.  Each thread loads 4 pieces of 16 bytes
// of a chunk (8 adjacent threads cover the 128 bytes of one row), kGramDepth
// chunks ahead, into registers, and writes a chunk to one of two LDS buffers
// just before it is used; then wave w adds the chunk's products to the tiles
// (w, t), t < d / 32, of 32 x 32 with v_mfma_f32_32x32x16_bf16: in step s (16
// columns) lane l's operand is piece 2 s + l / 32 of row l mod 32 of a 32-row
// group.  Piece q of row r sits at position q ^ ((r / 2) mod 8) of the row in
// LDS, so the 16 rows that one operand read serves at a time hit every bank
// once.  Columns past the slice are zero.  The barrier between chunks orders
// LDS only: the loads of later chunks stay in flight across it.
constexpr int kGramChunk = 64;  // columns per LDS chunk: 8 pieces of 16 bytes a row
#ifndef QKVNR_GRAM_DEPTH
#define QKVNR_GRAM_DEPTH 2
#endif
constexpr int kGramDepth = QKVNR_GRAM_DEPTH;  // chunks in flight per thread
static_assert(kGramDepth >= 2 && kGramDepth % 2 == 0 && kGramDepth <= 8, "even Gram prefetch depth 2..8");

template <int D>
__global__ __launch_bounds__(kWave * (D / 32)) void gram_partials_kernel(const uint16_t* __restrict__ x, int cols,
                                                                        int slice, float* __restrict__ out) {
  constexpr int T = D / 32, THREADS = kWave * T, PIECES = kGramChunk / 8;
  constexpr int PER = D * PIECES / THREADS;  // pieces each thread loads per chunk (4)
  __shared__ uint4 lds[2][D * PIECES];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t blk = blockIdx.x;
  const int part = blockIdx.y, parts = gridDim.y;
  const int k0 = part * slice, kend = min(cols, k0 + slice);
  const int chunks = kend > k0 ? (kend - k0 + kGramChunk - 1) / kGramChunk : 0;
  const int q = threadIdx.x % PIECES;
  const uint16_t* rp[PER];
  int slot[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = (threadIdx.x + j * THREADS) / PIECES;
    rp[j] = x + (blk * D + r) * cols;
    slot[j] = r * PIECES + (q ^ ((r >> 1) & 7));
  }
  auto load = [&](int c, uint4 (&v)[PER]) {
    const int col = min(k0 + c * kGramChunk + 8 * q, kend - 8);  // past the slice: its last columns again (cached)
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = ld16(rp[j] + col);
  };
  auto store = [&](int c, const uint4 (&v)[PER], uint4* buf) {
    // zero past the slice with a mask, not a branch (a branch here makes the compiler wait for every load)
    const uint32_t m = k0 + c * kGramChunk + 8 * q < kend ? 0xffffffffu : 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) buf[slot[j]] = make_uint4(v[j].x & m, v[j].y & m, v[j].z & m, v[j].w & m);
  };
  const int rr = lane % 32, h = lane / 32, sw = (rr >> 1) & 7;  // rows 32 t + rr share the swizzle
  f32x16_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x16_t{};
  constexpr int STEPS = kGramChunk / 16;
  uint4 a[STEPS], b[STEPS][T];
  auto reads = [&](const uint4* buf) {  // every operand of the chunk: one LDS round trip, not one a step
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int pos = (2 * st + h) ^ sw;
      a[st] = buf[(32 * w + rr) * PIECES + pos];
#pragma unroll
      for (int t = 0; t < T; ++t) b[st][t] = buf[(32 * t + rr) * PIECES + pos];
    }
  };
  auto mfmas = [&](int st) {
#pragma unroll
    for (int t = 0; t < T; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[st]),
                                                       __builtin_bit_cast(bf16x8_t, b[st][t]), acc[t], 0, 0, 0);
  };
  auto lds_barrier = [] {  // orders LDS only: later chunks' loads stay in flight across it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  // chunk c is loaded into v[c mod depth] (in chunk order, so that each store waits for its own
  // chunk only), stored to LDS buffer c mod 2 one chunk ahead of its products, and the store and
  // the next loads are issued between the products of the chunk before, while the matrix unit works
  uint4 v[kGramDepth][PER];
#pragma unroll
  for (int j = 0; j < kGramDepth; ++j) {
    load(j, v[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  store(0, v[0], lds[0]);
  load(kGramDepth, v[0]);
  lds_barrier();
  for (int c0 = 0; c0 < chunks; c0 += kGramDepth) {
#pragma unroll
    for (int j = 0; j < kGramDepth; ++j) {
      // loads, stores and barriers on every path (chunks past the slice are zeros); products for
      // chunks of the slice only (the same for the whole workgroup)
      const int c = c0 + j;
      const bool live = c < chunks;
      if (live) {
        reads(lds[j & 1]);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      store(c + 1, v[(j + 1) % kGramDepth], lds[(j + 1) & 1]);
      load(c + 1 + kGramDepth, v[(j + 1) % kGramDepth]);
      __builtin_amdgcn_sched_barrier(0);
      if (live) {
#pragma unroll
        for (int st = 1; st < STEPS; ++st) mfmas(st);
      }
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
    }
  }
  // C register e of lane l is row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32 of the tile
  float* o = out + (blk * parts + part) * D * D;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      o[(32 * w + 8 * (e / 4) + 4 * h + e % 4) * D + 32 * t + rr] = acc[t][e];
}

// P from the Gram matrix A of each block (the sum of its partials, at
// gram + b * parts * d * d): one workgroup per (block, group of 32 rows of P).
// The workgroup adds the partials into LDS and forms its rows of A^2 in 4 x 4
// patches (A is symmetric, so both factors are read along rows of A, 16 bytes
// at a time).
// DT > 0 fixes d at compile time (the common side 128); 0 takes it from `d_rt`.
template <typename OUT, int DT>
__global__ __launch_bounds__(kNsThreads) void ns_poly_kernel(const float* __restrict__ gram, OUT* __restrict__ out,
                                                            int d_rt, int parts, int first, float last_scale,
                                                            float eps) {
  const int d = DT > 0 ? DT : d_rt;
  constexpr int LD = kNsMaxD + 4;  // rows 16-byte aligned for float4 reads
  __shared__ __align__(16) float A[kNsMaxD * LD];
  __shared__ float red[kNsThreads / kWave];
  const int64_t blk = blockIdx.x;
  const int row0 = blockIdx.y * 32, rows = min(32, d - row0);
  const float* g = gram + blk * parts * d * d;
  if (d % 4 == 0) {  // 16-byte loads (a row holds whole groups of 4); each part's loads go out before they are added
    constexpr int CH = kNsMaxD * kNsMaxD / 4 / kNsThreads;
    const int n4 = d * d / 4;
    const float4* g4 = reinterpret_cast<const float4*>(g);
    float4 v[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = threadIdx.x + j * kNsThreads;
      v[j] = i < n4 ? g4[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    for (int pt = 1; pt < parts; ++pt) {  // partials added in order
      float4 u[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int i = threadIdx.x + j * kNsThreads;
        u[j] = i < n4 ? g4[static_cast<int64_t>(pt) * n4 + i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
#pragma unroll
      for (int j = 0; j < CH; ++j) v[j] = make_float4(v[j].x + u[j].x, v[j].y + u[j].y, v[j].z + u[j].z, v[j].w + u[j].w);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = 4 * (threadIdx.x + j * kNsThreads);
      if (i < d * d) *reinterpret_cast<float4*>(&A[(i / d) * LD + i % d]) = v[j];
    }
  } else {  // one value at a time
    const int n = d * d;
    for (int i = threadIdx.x; i < n; i += kNsThreads) {
      float a = g[i];
      for (int pt = 1; pt < parts; ++pt) a += g[static_cast<int64_t>(pt) * n + i];
      A[(i / d) * LD + i % d] = a;
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
    // A is symmetric, so both factors of (A^2)[r][c] = sum_k A[r][k] A[k][c] are read along row k,
    // 4 adjacent values at a time (past column d they are never stored into P)
#pragma unroll 4
    for (int k = 0; k < d; ++k) {
      const float4 r4 = *reinterpret_cast<const float4*>(&A[k * LD + r0]);
      const float4 c4 = *reinterpret_cast<const float4*>(&A[k * LD + c0]);
      const float ar[4] = {r4.x, r4.y, r4.z, r4.w}, ac[4] = {c4.x, c4.y, c4.z, c4.w};
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

// One Newton-Schulz update of bf16 blocks, Y = P X, and (GRAM) the partial Gram matrices of Y
// that the next step needs, from the same pass over X: Y is written once and never read back.
// p [blocks, D, D] bf16, x and y [blocks, D, cols] bf16 (row stride cols), gout [blocks, parts,
// D, D] fp32 over the column slices of gram_partials_kernel.  One workgroup per (block, slice),
// D / 32 waves, chunks of 64 columns:
// - X's chunk is loaded into registers three chunks ahead, thread (rg, cg) holding rows
//   4 rg + [0, 4) of columns 8 cg + [0, 8), and written to LDS transposed (X^T, rows of D values
//   along k): column n's 4 values go to piece k / 8 of row n at position (k / 8) ^ (n mod D/8);
// - the product is taken as Y^T = X^T P^T: the A operand is a row of X^T and the B operand a row
//   of P, so P needs no transpose, and each lane keeps its P operands in registers for the whole
//   slice.  Wave w forms rows 32 w + [0, 32) of Y for the chunk's 64 columns;
// - Y is rounded to bf16 into LDS in the Gram layout (piece q of row r at q ^ ((r / 2) mod 8);
//   columns past the slice are zero), then stored with 16-byte writes and, for GRAM, its chunk
//   products are added as in gram_partials_kernel.
// Software pipelined, one barrier a chunk: between two barriers a wave forms chunk c's product
// (from X^T buffer c mod 2), stores and adds the Gram products of chunk c - 1 (Y buffer
// (c - 1) mod 2), writes chunk c + 1's X^T and then chunk c's Y.  A buffer is rewritten only
// after the barrier that follows its last reads.  64 KB of LDS: two workgroups fit on a CU.
template <int D, bool GRAM>
__global__ __launch_bounds__(kWave * (D / 32), 2) void ns_update_kernel(const uint16_t* __restrict__ p,
                                                                       const uint16_t* __restrict__ x,
                                                                       uint16_t* __restrict__ y, int cols, int slice,
                                                                       float* __restrict__ gout) {
  static_assert(D == 64 || D == 128, "block sides 64 and 128");
  constexpr int T = D / 32, THREADS = kWave * T;
  constexpr int XP = D / 8;                  // 16-byte pieces of an X^T row
  constexpr int YP = kGramChunk / 8;         // 16-byte pieces of a Y row
  constexpr int KS = D / 16;                 // MFMA steps over k for the product
  static_assert(THREADS == 2 * D, "one thread per 4 x 8 patch of a chunk");
  __shared__ uint4 xt[2][kGramChunk * XP];
  __shared__ uint4 ys[2][D * YP];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int64_t blk = blockIdx.x;
  const int part = blockIdx.y, parts = gridDim.y;
  const int k0 = part * slice, kend = min(cols, k0 + slice);
  const int chunks = kend > k0 ? (kend - k0 + kGramChunk - 1) / kGramChunk : 0;
  const int rr = lane % 32, h = lane / 32;

  // P operands of this lane: row 32 w + rr, k = 16 s + 8 h + [0, 8)
  uint4 pf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) pf[s] = ld16(p + (blk * D + 32 * w + rr) * D + 16 * s + 8 * h);

  const int rg = threadIdx.x / 8, cg = threadIdx.x % 8;
  const uint16_t* xr = x + (blk * D + 4 * rg) * static_cast<int64_t>(cols);
  auto load = [&](int c, uint4 (&v)[4]) {
    const int col = min(k0 + c * kGramChunk + 8 * cg, kend - 8);  // past the slice: its last columns again (cached)
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld16(xr + static_cast<int64_t>(i) * cols + col);
  };
  auto dword = [](const uint4& u, int d) { return d == 0 ? u.x : (d == 1 ? u.y : (d == 2 ? u.z : u.w)); };
  auto store_xt = [&](const uint4 (&v)[4], uint4* buf) {
    const int k = 4 * rg;
#pragma unroll
    for (int d = 0; d < 4; ++d) {  // dword d of a row holds columns 2 d (low half) and 2 d + 1
      const uint32_t a0 = dword(v[0], d), a1 = dword(v[1], d), a2 = dword(v[2], d), a3 = dword(v[3], d);
      const uint2 lo = make_uint2((a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16));
      const uint2 hi = make_uint2((a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u));
      const int n0 = 8 * cg + 2 * d, n1 = n0 + 1;
      reinterpret_cast<uint2*>(&buf[n0 * XP + ((k >> 3) ^ (n0 & (XP - 1)))])[(k >> 2) & 1] = lo;
      reinterpret_cast<uint2*>(&buf[n1 * XP + ((k >> 3) ^ (n1 & (XP - 1)))])[(k >> 2) & 1] = hi;
    }
  };
  auto lds_barrier = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  const int sw = (rr >> 1) & 7;  // Gram layout swizzle of rows 32 t + rr
  f32x16_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x16_t{};

  auto product = [&](const uint4* xb, f32x16_t (&ya)[2]) {  // Y^T of the chunk's two 32-column tiles
    ya[0] = ya[1] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int n = 32 * ni + rr;
        const uint4 af = xb[n * XP + ((2 * s + h) ^ (n & (XP - 1)))];
        ya[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af),
                                                         __builtin_bit_cast(bf16x8_t, pf[s]), ya[ni], 0, 0, 0);
      }
  };
  // lane (rr, h) holds Y[32 w + rr][32 ni + 8 q + 4 h + r] in register 4 q + r of ya[ni]
  auto write_y = [&](int c, const f32x16_t (&ya)[2], uint4* yb) {
    const int cbase = k0 + c * kGramChunk, m = 32 * w + rr;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int piece = 4 * ni + q;
        const bool in = cbase + 8 * piece < kend;
        const uint2 val = in ? make_uint2(pack_bf16x2(ya[ni][4 * q], ya[ni][4 * q + 1]),
                                          pack_bf16x2(ya[ni][4 * q + 2], ya[ni][4 * q + 3]))
                             : make_uint2(0u, 0u);
        reinterpret_cast<uint2*>(&yb[m * YP + (piece ^ ((m >> 1) & 7))])[h] = val;
      }
  };
  auto finish = [&](int c, const uint4* yb) {  // chunk c's stores and Gram products, from its Y buffer
    const int cbase = k0 + c * kGramChunk;
#pragma unroll
    for (int j = 0; j < D * YP / THREADS; ++j) {
      const int u = threadIdx.x + j * THREADS, row = u / YP, q = u % YP;
      const int col = cbase + 8 * q;
      if (col < kend) st16(y + (blk * D + row) * static_cast<int64_t>(cols) + col, yb[row * YP + (q ^ ((row >> 1) & 7))]);
    }
    if constexpr (GRAM) {
#pragma unroll
      for (int st = 0; st < kGramChunk / 16; ++st) {
        const int pos = (2 * st + h) ^ sw;
        const uint4 a = yb[(32 * w + rr) * YP + pos];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint4 b = yb[(32 * t + rr) * YP + pos];
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, b), acc[t], 0, 0, 0);
        }
      }
    }
  };
  // phase c: the loads, LDS writes and barrier run on every path; the products, stores and Gram
  // products only for chunks of the slice (the same for the whole workgroup)
  auto phase = [&](int c, uint4 (&vn)[4], int b) {
    f32x16_t ya[2];
    if (c < chunks) product(xt[b], ya);
    if (c >= 1 && c - 1 < chunks) finish(c - 1, ys[b ^ 1]);
    store_xt(vn, xt[b ^ 1]);  // chunk c + 1
    load(c + 3, vn);
    if (c < chunks) write_y(c, ya, ys[b]);
    lds_barrier();
  };
  // chunk c + 1 is in v[(c + 1) mod 2] when phase c starts
  uint4 v0[4], v1[4];
  load(0, v0);
  load(1, v1);
  store_xt(v0, xt[0]);
  load(2, v0);
  lds_barrier();
  for (int c0 = 0; c0 < chunks; c0 += 2) {
    phase(c0, v1, 0);
    phase(c0 + 1, v0, 1);
  }
  // the last chunk's stores and Gram products: the loop's phase c = chunks has done them unless
  // chunks is even, where the loop ends at c = chunks - 1
  if (chunks > 0 && chunks % 2 == 0) finish(chunks - 1, ys[(chunks - 1) & 1]);
  if constexpr (GRAM) {
    float* o = gout + (blk * parts + part) * D * D;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        o[(32 * w + 8 * (e / 4) + 4 * h + e % 4) * D + 32 * t + rr] = acc[t][e];
  }
}

}  // namespace qkvnr
