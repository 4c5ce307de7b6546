// The QKV projection with the region fused into its epilogue.
//
// torchtitan page "[muse_spark][perf] Split the packed qkv inside the q/k
// region": the region's input is the packed output of the attention's QKV
// projection (Problem, item 1), and the page measures the region with the GEMMs
// left out (Results).  Here the region runs in the projection's epilogue: the
// packed product x w_qkv^T is formed with MFMA in fp32 and never written; each
// head of it is split out, q and k get the per-head RMSNorm and RoPE of the
// region, v is rounded, and q, k, v are stored as the region's forward stores
// them.  Only the final q/k/v writes reach memory (the packed write and its
// re-read are gone), and the packed values are never rounded to bf16.
//
// The product is a plain NT GEMM: x [T, hidden] and w_qkv [width, hidden] are
// both read along hidden.  Workgroup tile: 256 tokens x 256 packed columns (2
// heads of 128 or 4 of 64, so every head of the tile is whole), hidden in steps
// of 64, two LDS stages of 2 x 32 KB.  Four waves of 128 x 128.  The products
// are taken transposed, C^T = w x^T (v_mfma_f32_32x32x16_bf16 with the weight
// rows as the first operand): register e of lane l then holds packed column
// 8 (e / 4) + 4 (l / 32) + e % 4 of its 32-column tile for token l mod 32, so a
// lane owns 4 adjacent values of a head for each of its tokens.  A head's sum of
// squares is the lane's own sum plus one exchange with lane l ^ 32, and the
// rotate-half partner of a value is in the same lane, 64 (or 32) columns on.
#pragma once

#include "device.h"

namespace qkvnr {

typedef __bf16 pbf16x8_t __attribute__((ext_vector_type(8)));
typedef float pf32x16_t __attribute__((ext_vector_type(16)));

constexpr int kProjBM = 256, kProjBN = 256, kProjBK = 64;
constexpr int kProjThreads = 256;
constexpr int kProjMaxPairs = 64;

struct ProjArgs {
  const uint16_t* x;     // [T, hidden]
  const uint16_t* w;     // [width, hidden]
  const int32_t* pos;    // [T]
  const uint16_t* wq;    // [D]
  const uint16_t* wk;    // [D]
  uint16_t* q;           // [T, n_q, D]
  uint16_t* k;           // [T, n_kv, D]
  uint16_t* v;           // [T, n_kv, D]
  int64_t T;
  int32_t hidden;
  int32_t width;         // (n_q + 2 n_kv) D
  int32_t tiles_n;       // ceil(width / 256)
  int32_t kind;          // 0 interleaved, 1 sectioned
  int32_t n_kv;
  int32_t q_per_kv;
  int32_t n_q;
  int32_t heads;         // n_q + 2 n_kv
  float eps;
  double turns[kProjMaxPairs];  // turns per position of rotate-half pair i: theta^(-2i/R) / (2 pi)
};

// Which output a packed head block is: type 0 = q, 1 = k, 2 = v, and its head index there.
__device__ __forceinline__ void proj_head(const ProjArgs& a, int h, int& type, int& idx) {
  if (a.kind == 0) {
    const int g = h / (a.q_per_kv + 2), s = h - g * (a.q_per_kv + 2);
    type = s < a.q_per_kv ? 0 : (s == a.q_per_kv ? 1 : 2);
    idx = type == 0 ? g * a.q_per_kv + s : g;
  } else {
    type = h < a.n_q ? 0 : (h < a.n_q + a.n_kv ? 1 : 2);
    idx = h - (type == 0 ? 0 : (type == 1 ? a.n_q : a.n_q + a.n_kv));
  }
}

template <int D, bool ROPE>
__global__ __launch_bounds__(kProjThreads, 1) void proj_qkv_kernel(const ProjArgs a) {
  constexpr int PIECES = kProjBK / 8;       // 16-byte pieces of a row per K step
  constexpr int ROWS = kProjBM * PIECES;    // pieces of one operand tile
  constexpr int PER = kProjBM / (kProjThreads / PIECES);  // rows each thread loads per operand (8)
  __shared__ uint4 lds[2][2][ROWS];         // [stage][x, w][row * 8 + swizzled piece]: 128 KB
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = w >> 1, wn = w & 1;
  const int tn = blockIdx.x % a.tiles_n;
  const int64_t tm = blockIdx.x / a.tiles_n;
  const int64_t m0 = tm * kProjBM;
  const int n0 = tn * kProjBN;

  // ---- operand loads: thread t loads piece t mod 8 of rows t / 8 + 32 j (rows past the end clamped)
  const int q = threadIdx.x % PIECES;
  const uint16_t* pa[PER];
  const uint16_t* pb[PER];
  int slot[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = threadIdx.x / PIECES + (kProjThreads / PIECES) * j;
    pa[j] = a.x + min<int64_t>(m0 + r, a.T - 1) * a.hidden + 8 * q;
    pb[j] = a.w + static_cast<int64_t>(min(n0 + r, a.width - 1)) * a.hidden + 8 * q;
    slot[j] = r * PIECES + (q ^ ((r >> 1) & 7));  // the 16 rows one operand read serves hit every bank once
  }
  uint4 sa[PER], sb[PER];
  auto gload = [&](int kt) {
    const int off = kt * kProjBK;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      sa[j] = ld16(pa[j] + off);
      sb[j] = ld16(pb[j] + off);
    }
  };
  auto lstore = [&](int stage) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      lds[stage][0][slot[j]] = sa[j];
      lds[stage][1][slot[j]] = sb[j];
    }
  };
  auto lds_barrier = [] {  // orders LDS only: the next step's loads stay in flight across it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  // ---- MFMA fragments: step s of a K step, lane l reads piece 2 s + l / 32 of row l mod 32 of a 32-row group
  const int rr = lane % 32, h = lane / 32, sw = (rr >> 1) & 7;
  pf32x16_t acc[4][4];  // [packed 32-column tile j][token tile i]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = pf32x16_t{};
  uint4 fa[2][4], fb[2][4];
  auto reads = [&](int stage, int s, uint4 (&xa)[4], uint4 (&xb)[4]) {
    const int pos = (2 * s + h) ^ sw;
#pragma unroll
    for (int i = 0; i < 4; ++i) xa[i] = lds[stage][0][(128 * wm + 32 * i + rr) * PIECES + pos];
#pragma unroll
    for (int j = 0; j < 4; ++j) xb[j] = lds[stage][1][(128 * wn + 32 * j + rr) * PIECES + pos];
  };
  auto mfmas = [&](const uint4 (&xa)[4], const uint4 (&xb)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pbf16x8_t, xb[j]),
                                                            __builtin_bit_cast(pbf16x8_t, xa[i]), acc[j][i], 0, 0, 0);
  };

  const int KT = a.hidden / kProjBK;
  gload(0);
  lstore(0);
  gload(min(1, KT - 1));
  lds_barrier();
  for (int kt = 0; kt < KT; ++kt) {
    const int stage = kt & 1;
    // step kt + 1 goes to the other stage (last read before the previous barrier) during this step's
    // products; the load of step kt + 2 follows it (past the end it reloads the last step, unused)
    reads(stage, 0, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    reads(stage, 1, fa[1], fb[1]);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    lstore(stage ^ 1);
    gload(min(kt + 2, KT - 1));
    __builtin_amdgcn_sched_barrier(0);
    reads(stage, 2, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa[1], fb[1]);
    __builtin_amdgcn_sched_barrier(0);
    reads(stage, 3, fa[1], fb[1]);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa[1], fb[1]);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  }

  // ---- epilogue.  Lane (rr, h) holds, for token 128 wm + 32 i + rr and packed tile j, the columns
  // 128 wn + 32 j + 8 c + 4 h + r in register 4 c + r.  A head is D / 32 consecutive tiles j.
  constexpr int TPH = D / 32;              // tiles per head
  constexpr int HPW = 4 / TPH;             // heads per wave
  const int hb0 = (n0 + 128 * wn) / D;     // first packed head of this wave
  float wv[HPW][TPH][16];                  // norm weight of each held column (per head type)
  int type[HPW], idx[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    proj_head(a, min(hb0 + hh, a.heads - 1), type[hh], idx[hh]);
    const uint16_t* wsrc = type[hh] == 0 ? a.wq : a.wk;
#pragma unroll
    for (int jj = 0; jj < TPH; ++jj)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        wv[hh][jj][e] = type[hh] == 2 ? 1.0f
                                      : __builtin_bit_cast(float, static_cast<uint32_t>(wsrc[32 * jj + 8 * (e / 4) + 4 * h + e % 4]) << 16);
  }
  const float inv_d = 1.0f / D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = m0 + 128 * wm + 32 * i + rr;
    float ss[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float s = 0.0f;
#pragma unroll
      for (int jj = 0; jj < TPH; ++jj)
#pragma unroll
        for (int e = 0; e < 16; ++e) s = fmaf(acc[hh * TPH + jj][i][e], acc[hh * TPH + jj][i][e], s);
      ss[hh] = s + __shfl_xor(s, 32, kWave);  // the other half of the head's columns
    }
    if constexpr (ROPE) {
      // cos / sin of pair p = 32 jj + 8 c + 4 h + r (jj < TPH / 2) at this token's position
      const int32_t p = a.pos[min<int64_t>(t, a.T - 1)];
      float cs[TPH / 2][16], sn[TPH / 2][16];
#pragma unroll
      for (int jj = 0; jj < TPH / 2; ++jj)
#pragma unroll
        for (int e = 0; e < 16; ++e) rope_cos_sin(p, a.turns[32 * jj + 8 * (e / 4) + 4 * h + e % 4], cs[jj][e], sn[jj][e]);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        if (type[hh] == 2) continue;
        const float r = rsqrtf(fmaf(ss[hh], inv_d, a.eps));
#pragma unroll
        for (int jj = 0; jj < TPH / 2; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float nl = acc[hh * TPH + jj][i][e] * r * wv[hh][jj][e];
            const float nh = acc[hh * TPH + jj + TPH / 2][i][e] * r * wv[hh][jj + TPH / 2][e];
            acc[hh * TPH + jj][i][e] = nl * cs[jj][e] - nh * sn[jj][e];
            acc[hh * TPH + jj + TPH / 2][i][e] = nh * cs[jj][e] + nl * sn[jj][e];
          }
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        if (type[hh] == 2) continue;
        const float r = rsqrtf(fmaf(ss[hh], inv_d, a.eps));
#pragma unroll
        for (int jj = 0; jj < TPH; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[hh * TPH + jj][i][e] = acc[hh * TPH + jj][i][e] * r * wv[hh][jj][e];
      }
    }
  }

  // ---- bf16 tile through LDS (the operand stages are free after the last barrier), then rows out.
  // Staging row = token of the tile, 32 granules of 16 bytes; granule g of row r sits at g ^ (r mod 32).
  uint4* st = &lds[0][0][0];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 128 * wm + 32 * i + rr;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int g = 16 * wn + 4 * j + c;
        uint2* dst = reinterpret_cast<uint2*>(st + row * 32 + (g ^ (row & 31))) + h;
        *dst = make_uint2(pack_bf16x2(acc[j][i][4 * c], acc[j][i][4 * c + 1]),
                          pack_bf16x2(acc[j][i][4 * c + 2], acc[j][i][4 * c + 3]));
      }
  }
  __syncthreads();
  // 256 rows x 32 granules; thread t takes granule t mod 32 of rows t / 32 + 8 u
#pragma unroll 4
  for (int u = 0; u < kProjBM / 8; ++u) {
    const int row = threadIdx.x / 32 + 8 * u, g = threadIdx.x % 32;
    const int64_t t = m0 + row;
    const int col = n0 + 8 * g;            // packed column of the granule
    const int hb = col / D;
    if (t < a.T && hb < a.heads) {
      int ty, ix;
      proj_head(a, hb, ty, ix);
      uint16_t* base = ty == 0 ? a.q : (ty == 1 ? a.k : a.v);
      const int nh = ty == 0 ? a.n_q : a.n_kv;
      st16(base + (t * nh + ix) * D + col % D, st[row * 32 + (g ^ (row & 31))]);
    }
  }
}

}  // namespace qkvnr
