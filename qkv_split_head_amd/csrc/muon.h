// Per-head Newton-Schulz on fused QKV weights: the per-block steps, and the steps collapsed.
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
// and P by the norm) and the last step's scale; the update P X is
// ns_update_kernel (bf16 blocks of side 64 and 128) or a batched GEMM.
//
// For bf16 blocks of side 64 and 128 the steps are also collapsed into one d x d
// matrix M per block (ns_collapse_kernel, from the Gram partials of G), and the
// result is M G in one more pass (ns_update_kernel<SPLIT>).
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
//   along k): column n's 4 values go to piece k / 8 of row n at position (k / 8) ^ xswz(n);
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
//
// SPLIT: p holds two bf16 terms per block, [blocks][2][D][D] (hi, then lo), and Y = (hi + lo) X: two
// products a step, added in fp32 before Y's one rounding (the collapsed iteration's M, whose terms
// carry about 16 bits).
template <int D, bool GRAM, bool SPLIT = false>
__global__ __launch_bounds__(kWave * (D / 32), 2) void ns_update_kernel(const uint16_t* __restrict__ p,
                                                                       const uint16_t* __restrict__ x,
                                                                       uint16_t* __restrict__ y, int cols, int slice,
                                                                       float* __restrict__ gout) {
  static_assert(D == 64 || D == 128, "block sides 64 and 128");
  static_assert(!(GRAM && SPLIT), "the split product forms no Gram matrices");
  constexpr int T = D / 32, THREADS = kWave * T;
  constexpr int XP = D / 8;                  // 16-byte pieces of an X^T row
  constexpr int YP = kGramChunk / 8;         // 16-byte pieces of a Y row
  constexpr int KS = D / 16;                 // MFMA steps over k for the product
  static_assert(THREADS == 2 * D, "one thread per 4 x 8 patch of a chunk");
  __shared__ uint4 xt[2][kGramChunk * XP];
  __shared__ uint4 ys[2][D * YP];
  // X^T row n's piece q sits at q ^ xswz(n).  A write instruction covers columns n = 8 cg + c (c fixed) of
  // 8 consecutive k rows: for D = 128 the swizzle mixes n's bits 4-5 into bits 1-2 as well as taking n mod 16,
  // so those lanes hit 32 bank pairs twice each (n mod 16 alone takes 2 values there: 4 lanes a pair); each
  // 16 lanes of an operand read (16 consecutive n) still hit 16 different pieces.
  auto xswz = [](int n) {
    if constexpr (XP == 16) return (n & 15) ^ (((n >> 4) & 3) << 1);
    else return n & (XP - 1);
  };
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int64_t blk = blockIdx.x;
  const int part = blockIdx.y, parts = gridDim.y;
  const int k0 = part * slice, kend = min(cols, k0 + slice);
  const int chunks = kend > k0 ? (kend - k0 + kGramChunk - 1) / kGramChunk : 0;
  const int rr = lane % 32, h = lane / 32;

  // P operands of this lane: row 32 w + rr, k = 16 s + 8 h + [0, 8)
  uint4 pf[KS], pl[SPLIT ? KS : 1];
  const uint16_t* prow = p + (blk * (SPLIT ? 2 : 1) * D + 32 * w + rr) * D + 8 * h;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    pf[s] = ld16(prow + 16 * s);
    if constexpr (SPLIT) pl[s] = ld16(prow + D * D + 16 * s);
  }

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
      reinterpret_cast<uint2*>(&buf[n0 * XP + ((k >> 3) ^ xswz(n0))])[(k >> 2) & 1] = lo;
      reinterpret_cast<uint2*>(&buf[n1 * XP + ((k >> 3) ^ xswz(n1))])[(k >> 2) & 1] = hi;
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
        const uint4 af = xb[n * XP + ((2 * s + h) ^ xswz(n))];
        if constexpr (SPLIT)
          ya[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af),
                                                           __builtin_bit_cast(bf16x8_t, pl[s]), ya[ni], 0, 0, 0);
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

// The iteration collapsed into one d x d computation per block.  Every step multiplies X by a
// polynomial in the block's Gram matrix, and every such polynomial commutes with A0 = G G^T, so
// the iterate after k steps is X_k = M_k X_0 with M_k a polynomial in A0: with A'_0 = A0 / (n + eps)^2
// (n^2 = trace A0 = ||G||_F^2),
//   P_k = 3.4445 I - 4.7750 A'_k + 2.0315 A'_k A'_k,   A'_{k+1} = P_k A'_k P_k,   M_{k+1} = P_k M_k,
// and the result is M G with M = M_steps scale / (n + eps): the same function of G as the steps
// taken on X (ns_poly_kernel and the update), with two passes over G (its Gram matrix, then M G)
// instead of two a step.  Every matrix here is a polynomial in A0, hence symmetric, which the
// products use: product(a, b) takes tiles of a b^T, rows 32 t + [0, 32) of a (A operand) against a
// wave's 32 rows of b (B operand), and reads them transposed, as rows of b a^T: each wave then holds
// rows of every result, in the pieces that its LDS writes need.
// Precision: every factor is held as two bf16 terms, hi = bf16(v) and lo = bf16(v - hi) (within
// 2^-16 |v|), and every product is hi hi + hi lo + lo hi with fp32 accumulation (within about 2^-14
// of |a| |b|); M goes out in the same two terms, applied as (hi + lo) G by ns_update_kernel<SPLIT>.
// One bf16 rounding of M (2^-9 relative) would not do: M's entries grow with the block's condition
// while M G stays near orthogonal, so its rounding errors do not cancel.
// One workgroup per block, ns_collapse_waves(D) waves: wave w owns rows 32 (w mod D/32) + [0, 32) and
// its group of column tiles of every result.  LDS: two regions of a D x D matrix each as hi and lo, in
// gram_partials_kernel's layout (chunks of 64 columns, row r's 16-byte piece j at j ^ ((r / 2) mod 8)):
// rp holds P_k, ra holds A'_k, then P_k A'_k, then M_k while M_{k+1} is formed.
//
// Waves of the collapse kernel: D / 32 row bands times up to QKVNR_NS_CSPLIT groups of column tiles, one
// tile a wave by default (16 waves for D = 128, four a SIMD: 45 us for 48 blocks of 128, against 47 us with
// two tiles a wave and 65 us with four).
#ifndef QKVNR_NS_CSPLIT
#define QKVNR_NS_CSPLIT 4
#endif
constexpr int ns_collapse_waves(int d) { return (d / 32) * (QKVNR_NS_CSPLIT < d / 32 ? QKVNR_NS_CSPLIT : d / 32); }
template <int D>
__global__ __launch_bounds__(kWave * ns_collapse_waves(D), 1) void ns_collapse_kernel(const float* __restrict__ gram,
                                                                                     int parts, int steps,
                                                                                     float scale, float eps,
                                                                                     uint16_t* __restrict__ m) {
  static_assert(D == 64 || D == 128, "block sides 64 and 128");
  constexpr int T = D / 32, WAVES = ns_collapse_waves(D), TH = T * T / WAVES, THREADS = kWave * WAVES;
  constexpr int N = D * D, V = N / 4 / THREADS;
  constexpr int KS = D / 16;
  __shared__ uint4 ra[2][N / 8];  // A'_k, then P_k A'_k, then M_k: hi, lo
  __shared__ uint4 rp[2][N / 8];  // P_k: hi, lo
  __shared__ float tred[WAVES];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int rr = lane % 32, h = lane / 32, sw = (rr >> 1) & 7;
  const int r = 32 * (w % T) + rr, t0 = (w / T) * TH;  // this lane's row; this wave's first column tile
  const int64_t blk = blockIdx.x;
  auto lds_barrier = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  auto slot = [](int row, int col) { return (col >> 6) * D * 8 + row * 8 + (((col & 63) >> 3) ^ ((row >> 1) & 7)); };
  auto rest = [](float v, uint32_t pk, int upper) {  // v minus its bf16 value (the upper or lower half of pk)
    return v - __uint_as_float(upper ? (pk & 0xffff0000u) : (pk << 16));
  };
  // hi and lo of 4 adjacent values (row, col .. col + 3) into a region
  auto put = [&](uint4 (*reg)[N / 8], int row, int col, float4 v) {
    const uint2 hi = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    const uint2 lo = make_uint2(pack_bf16x2(rest(v.x, hi.x, 0), rest(v.y, hi.x, 1)),
                                pack_bf16x2(rest(v.z, hi.y, 0), rest(v.w, hi.y, 1)));
    reinterpret_cast<uint2*>(&reg[0][slot(row, col)])[(col >> 2) & 1] = hi;
    reinterpret_cast<uint2*>(&reg[1][slot(row, col)])[(col >> 2) & 1] = lo;
  };
  auto unpack4 = [](uint2 u, float (&f)[4]) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
  };
  // hi + lo of (row, col .. col + 3)
  auto get = [&](uint4 (*reg)[N / 8], int row, int col) {
    float a[4], b[4];
    unpack4(reinterpret_cast<const uint2*>(&reg[0][slot(row, col)])[(col >> 2) & 1], a);
    unpack4(reinterpret_cast<const uint2*>(&reg[1][slot(row, col)])[(col >> 2) & 1], b);
    return make_float4(a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]);
  };
  // product(a, b): tiles t0 + i of a b^T (rows 32 t of a against rows of b in this wave's band), each read
  // transposed: acc[i] register 4 e4 + j is (b a^T)[r][32 (t0 + i) + 8 e4 + 4 h + j].  Every operand is
  // hi + lo; hi hi + hi lo + lo hi, fp32 accumulation.
  auto product = [&](uint4 (*fa)[N / 8], uint4 (*fb)[N / 8], f32x16_t (&acc)[TH]) {
#pragma unroll
    for (int i = 0; i < TH; ++i) acc[i] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int base = (s / 4) * D * 8, pos = (2 * (s % 4) + h) ^ sw;
      const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, fb[0][base + r * 8 + pos]);
      const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, fb[1][base + r * 8 + pos]);
#pragma unroll
      for (int i = 0; i < TH; ++i) {
        const int ia = base + (32 * (t0 + i) + rr) * 8 + pos;
        const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, fa[0][ia]);
        const bf16x8_t al = __builtin_bit_cast(bf16x8_t, fa[1][ia]);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[i], 0, 0, 0);
      }
    }
  };
  auto col_of = [&](int i, int e4) { return 32 * (t0 + i) + 8 * e4 + 4 * h; };
  auto tile4 = [](const f32x16_t& a, int e4) { return make_float4(a[4 * e4], a[4 * e4 + 1], a[4 * e4 + 2], a[4 * e4 + 3]); };
  auto put_all = [&](uint4 (*reg)[N / 8], const float4 (&v)[TH][4]) {
#pragma unroll
    for (int i = 0; i < TH; ++i)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) put(reg, r, col_of(i, e4), v[i][e4]);
  };
  auto regs = [&](const f32x16_t (&acc)[TH], float4 (&v)[TH][4]) {
#pragma unroll
    for (int i = 0; i < TH; ++i)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) v[i][e4] = tile4(acc[i], e4);
  };

  // A0 = ((g0 + g1) + g2) + ...: thread x sums the 4 values at 4 (j THREADS + x), two slices in flight
  const float* g = gram + blk * parts * N;
  auto load = [&](int pt, float4 (&v)[V]) {
    const float4* src = reinterpret_cast<const float4*>(g + static_cast<int64_t>(pt) * N) + threadIdx.x;
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = src[j * THREADS];
  };
  auto add = [](float4 (&a)[V], const float4 (&b)[V]) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      a[j].x += b[j].x;
      a[j].y += b[j].y;
      a[j].z += b[j].z;
      a[j].w += b[j].w;
    }
  };
  float4 av[V];
  load(0, av);
  int pt = 1;
  for (; pt + 1 < parts; pt += 2) {
    float4 u0[V], u1[V];
    load(pt, u0);
    load(pt + 1, u1);
    add(av, u0);
    add(av, u1);
  }
  for (; pt < parts; ++pt) {
    float4 u0[V];
    load(pt, u0);
    add(av, u0);
  }
  // n^2 = trace A0 in a fixed order: each thread's diagonal values, the wave, then the waves
  float dg = 0.0f;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int u = 4 * (j * THREADS + static_cast<int>(threadIdx.x)), k = u / D - u % D;
    if (k >= 0 && k < 4) dg += k == 0 ? av[j].x : (k == 1 ? av[j].y : (k == 2 ? av[j].z : av[j].w));
  }
  for (int off = kWave / 2; off > 0; off >>= 1) dg += __shfl_xor(dg, off, kWave);
  if (lane == 0) tred[w] = dg;
  __syncthreads();
  float n2 = 0.0f;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) n2 += tred[i];
  const float norm_inv = 1.0f / (sqrtf(n2) + eps), a2s = norm_inv * norm_inv;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int u = 4 * (j * THREADS + static_cast<int>(threadIdx.x));
    put(ra, u / D, u % D, make_float4(av[j].x * a2s, av[j].y * a2s, av[j].z * a2s, av[j].w * a2s));
  }
  lds_barrier();

  float4 mr[TH][4];  // M_k: row r, this wave's columns
  f32x16_t acc[TH];
  for (int k = 0; k < steps; ++k) {
    // P_k = 3.4445 I - 4.7750 A' + 2.0315 A' A'
    product(ra, ra, acc);
    float4 pr[TH][4];
#pragma unroll
    for (int i = 0; i < TH; ++i)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int c = col_of(i, e4);
        const float4 a1 = get(ra, r, c), a2 = tile4(acc[i], e4);
        float4 pv = make_float4(fmaf(kNsC, a2.x, kNsB * a1.x), fmaf(kNsC, a2.y, kNsB * a1.y),
                                fmaf(kNsC, a2.z, kNsB * a1.z), fmaf(kNsC, a2.w, kNsB * a1.w));
        const int dd = r - c;  // the diagonal element of this row, if among these 4 columns
        if (dd == 0) pv.x += kNsA;
        if (dd == 1) pv.y += kNsA;
        if (dd == 2) pv.z += kNsA;
        if (dd == 3) pv.w += kNsA;
        pr[i][e4] = pv;
      }
    put_all(rp, pr);
    lds_barrier();
    float4 an[TH][4];
    if (k + 1 < steps) {
      // A'_{k+1} = (P_k A'_k) P_k.  The transposed reading makes product(a, b) = b a^T, so the factors go in
      // this order: another one (P_k P_k A'_k, say) is as good in exact arithmetic but not symmetric in
      // form, and its rounding's antisymmetric part would grow from step to step
      product(ra, rp, acc);  // P_k A'_k
      lds_barrier();         // every read of A'_k is done
      regs(acc, an);
      put_all(ra, an);
      lds_barrier();
      product(rp, ra, acc);  // (P_k A'_k) P_k
      regs(acc, an);
      lds_barrier();         // every read of P_k A'_k is done
    }
    if (k == 0) {
#pragma unroll
      for (int i = 0; i < TH; ++i)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) mr[i][e4] = pr[i][e4];
    } else {  // M_{k+1} = M_k P_k (= P_k M_k): rows of P against rows of M_k, staged in ra
      put_all(ra, mr);
      lds_barrier();
      product(rp, ra, acc);
      regs(acc, mr);
      lds_barrier();  // every read of M_k (and of P_k) is done
    }
    if (k + 1 < steps) {
      put_all(ra, an);
      lds_barrier();
    }
  }
  // M scale / (n + eps) as hi and lo: m + b 2 D D (hi) and + D D (lo), 8 bytes of each per (tile, e4)
  const float ms = scale * norm_inv;
  uint16_t* mh = m + blk * 2 * N + r * D;
#pragma unroll
  for (int i = 0; i < TH; ++i)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int c = col_of(i, e4);
      const float v[4] = {mr[i][e4].x * ms, mr[i][e4].y * ms, mr[i][e4].z * ms, mr[i][e4].w * ms};
      const uint2 hi = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      const uint2 lo = make_uint2(pack_bf16x2(rest(v[0], hi.x, 0), rest(v[1], hi.x, 1)),
                                  pack_bf16x2(rest(v[2], hi.y, 0), rest(v[3], hi.y, 1)));
      *reinterpret_cast<uint2*>(mh + c) = hi;
      *reinterpret_cast<uint2*>(mh + N + c) = lo;
    }
}

}  // namespace qkvnr
