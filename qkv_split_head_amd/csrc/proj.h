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
// of 64.  Two LDS stages of 2 x 32 KB are filled by direct-to-LDS loads one step
// ahead: a load has one step (64 MFMAs a wave) to return, and a step ends with
// one wait and one barrier.  Four waves of 128 x 128; the products are taken
// transposed, C^T = w x^T (v_mfma_f32_32x32x16_bf16 with the weight rows as the
// first operand), and the fragment reads and global loads of a step are spread
// one by one between its MFMAs.  Workgroups are persistent (one per CU) and take the tiles in a
// grouped order that keeps the tiles one XCD runs at once on shared rows.
// The epilogue moves each half of the tile to LDS as fp32 and finishes it the
// way the region's forward does: D / 16 threads per token head, a lane-group sum
// of squares, cos / sin of each thread's rotate-half pairs shared by the token's
// heads, and 16-byte stores of q, k and v.
#pragma once

#include "device.h"

namespace qkvnr {

typedef __bf16 pbf16x8_t __attribute__((ext_vector_type(8)));
typedef float pf32x16_t __attribute__((ext_vector_type(16)));

constexpr int kProjBM = 256, kProjBN = 256, kProjBK = 64;
constexpr int kProjStages = 2;  // LDS stages of one K step each: one loading while the other is read
constexpr int kProjThreads = 256;
constexpr int kProjGroupM = 4;  // token tiles per group of the tile order
static_assert(kProjThreads == kProjBM, "one thread per token of a tile fills the position table");
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
  int32_t tiles_m;       // ceil(T / 256)
  int32_t kind;          // 0 interleaved, 1 sectioned
  int32_t n_kv;
  int32_t q_per_kv;
  int32_t n_q;
  int32_t heads;         // n_q + 2 n_kv
  float eps;
  double turns[kProjMaxPairs];  // turns per position of rotate-half pair i: theta^(-2i/R) / (2 pi)
};

__device__ __forceinline__ float proj_bf16_f32(uint16_t b) { return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16); }

// Sum over an aligned group of G lanes (G = 4 or 8); every lane of the group gets the same bits.
template <int G>
__device__ __forceinline__ float proj_group_sum(float v) {
  if constexpr (G == 4) {
    v += dpp<kQuadXor1>(v);
    return v + dpp<kQuadXor2>(v);
  } else {
    return head_sum<G>(v);
  }
}

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

template <int D, bool ROPE, bool TAIL>
__global__ __launch_bounds__(kProjThreads, 1) void proj_qkv_kernel(const ProjArgs a) {
  constexpr int PIECES = kProjBK / 8;       // 16-byte pieces of a row per K step (8)
  constexpr int ROWS = kProjBM * PIECES;    // pieces of one operand tile (2048, 32 KB)
  // two stages of [x, w][row * 8 + swizzled piece], 64 KB each, as two arrays: with the stage of every
  // access known at compile time the compiler sees that reading one stage does not touch the other
  // while its direct-to-LDS loads are in flight
  __shared__ uint4 lds0[2][ROWS], lds1[2][ROWS];
  __shared__ uint16_t ep_w[2][D];           // q and k norm weights, for the epilogue
  __shared__ double ep_turns[D / 2];        // turns per position of each rotate-half pair
  __shared__ int32_t ep_pos[kProjBM];       // positions of the current tile's tokens
  if (threadIdx.x < D) {
    ep_w[0][threadIdx.x] = a.wq[threadIdx.x];
    ep_w[1][threadIdx.x] = a.wk[threadIdx.x];
    if (ROPE && threadIdx.x < D / 2) ep_turns[threadIdx.x] = a.turns[threadIdx.x];
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = w >> 1, wn = w & 1;

  // ---- persistent workgroups walk the tiles in rounds of gridDim.x.  Workgroup b runs on XCD
  // b mod 8, and in each round the XCD's workgroups take consecutive tiles of a grouped order
  // (kProjGroupM token tiles by every head tile), so the ones an XCD runs at once share operand
  // rows in its L2.
  const int P = gridDim.x;
  const int tiles = a.tiles_m * a.tiles_n;
  const int slot_in_round = P % 8 == 0 ? (blockIdx.x % 8) * (P / 8) + blockIdx.x / 8 : blockIdx.x;
  auto tile_of = [&](int L, int64_t& m0, int& n0) {
    const int group = L / (kProjGroupM * a.tiles_n), within = L % (kProjGroupM * a.tiles_n);
    const int gm = min(kProjGroupM, a.tiles_m - group * kProjGroupM);
    m0 = static_cast<int64_t>(group * kProjGroupM + within % gm) * kProjBM;
    n0 = (within / gm) * kProjBN;
  };

  // ---- operand loads, straight from global memory into an LDS stage (global_load_lds_dwordx4: lane
  // i of an instruction writes the 16 bytes at the instruction's LDS base + 16 i).  Per K step each
  // wave issues 16 of them: j < 8 for x, j >= 8 for the weight, instruction j covering the 8 rows
  // 8 (8 w + j % 8) + [0, 8) of its operand.  Lane i fills unit u = 64 (8 w + j % 8) + i of the
  // stage, row u / 8 position u % 8, so it loads the piece (u % 8) ^ swz(row) of that row (rows past
  // the end clamped): piece q of row r sits at position q ^ ((r / 2) mod 8), which puts the 16 rows
  // one fragment read serves on 16 different bank groups.
  const uint16_t* dsrc[16];
  auto dma_rows = [&](int64_t gm0, int gn0) {  // the sources' row starts for a tile (column 0, piece offset)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 8 * (8 * w + j % 8) + lane / 8;
      const int off = 8 * ((lane % 8) ^ ((r >> 1) & 7));
      dsrc[j] = j < 8 ? a.x + min<int64_t>(gm0 + r, a.T - 1) * a.hidden + off
                      : a.w + static_cast<int64_t>(min(gn0 + r, a.width - 1)) * a.hidden + off;
    }
  };
  auto dma = [&](uint4 (&stg)[2][ROWS], int kt) {  // K step kt of the current tile into a stage
#pragma unroll
    for (int j = 0; j < 16; ++j)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(dsrc[j] + kt * kProjBK),
                                       (__attribute__((address_space(3))) void*)(&stg[j / 8][64 * (8 * w + j % 8)]),
                                       16, 0, 0);
  };

  // ---- MFMA fragments: step s of a K step, lane l reads piece 2 s + l / 32 of row l mod 32 of a 32-row group
  const int rr = lane % 32, h = lane / 32, sw = (rr >> 1) & 7;
  pf32x16_t acc[4][4];  // [packed 32-column tile j][token tile i]
  uint4 fa[2][4], fb[2][4];  // fragments of alternate sub-steps of 16
  // Each lane's fragment row offsets are computed once and hidden from the optimiser, so every read
  // of a stage forms its address the same way: the waitcnt pass then still sees which stage a read
  // comes from (an address merged from two different forms costs a wait for every load in flight)
  int ia = (128 * wm + rr) * PIECES, ib = (128 * wn + rr) * PIECES;
  asm volatile("" : "+v"(ia), "+v"(ib));
  auto reads = [&](const uint4 (&stg)[2][ROWS], int s, uint4 (&xa)[4], uint4 (&xb)[4]) {
    const int pos = (2 * s + h) ^ sw;
#pragma unroll
    for (int i = 0; i < 4; ++i) xa[i] = stg[0][ia + 32 * i * PIECES + pos];
#pragma unroll
    for (int j = 0; j < 4; ++j) xb[j] = stg[1][ib + 32 * j * PIECES + pos];
  };
  auto mfmas = [&](const uint4 (&xa)[4], const uint4 (&xb)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pbf16x8_t, xb[j]),
                                                            __builtin_bit_cast(pbf16x8_t, xa[i]), acc[j][i], 0, 0, 0);
  };
  // Instruction order inside a K step, one MFMA at a time with the other work between them (the
  // scheduler is told the pattern, so no burst of reads or loads stalls the matrix unit): each
  // sub-step's 16 MFMAs have the next sub-step's 8 fragment reads between them, and the first
  // sub-step's also the 16 loads of the next K step.
  auto interleave = [](int reads, int writes, int vloads) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
      if (m < reads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      if (m < writes) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); // one LDS write
      if (m < vloads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // one global load
    }
  };

  constexpr int HEADS = kProjBN / D;          // heads per tile row
  constexpr int G = D / 16;                   // threads per token
  constexpr int TOK_PER_PASS = kProjThreads / G;
  const int k = threadIdx.x % G;
  const int KT = a.hidden / kProjBK;
  int L = slot_in_round;
  int64_t m0 = 0;
  int n0 = 0;
  __syncthreads();     // the epilogue tables above are complete
  // One K step: the next K step's loads go to the other stage (its last reads were before the last
  // barrier; past the tile's end they reload the last step, unused), the four sub-steps of 16 run
  // from the current stage, then every wave waits for its loads and meets the others at the barrier,
  // and sub-step 0 of the next stage is read.  Products only for steps of the tile.
  auto step = [&](const uint4 (&cur)[2][ROWS], uint4 (&nxt)[2][ROWS], int kt) {
    __builtin_amdgcn_sched_barrier(0);
    dma(nxt, min(kt + 1, KT - 1));
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if (s4 < 3) reads(cur, s4 + 1, fa[(s4 + 1) & 1], fb[(s4 + 1) & 1]);
      if (!TAIL || kt < KT) mfmas(fa[s4 & 1], fb[s4 & 1]);
      interleave(s4 < 3 ? 8 : 0, 0, s4 == 0 ? 16 : 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next K step has landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    reads(nxt, 0, fa[0], fb[0]);
  };
  for (; L < tiles; L += P) {
    tile_of(L, m0, n0);
    if (ROPE) ep_pos[threadIdx.x] = a.pos[min<int64_t>(m0 + threadIdx.x, a.T - 1)];  // kProjThreads == kProjBM
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = pf32x16_t{};
    dma_rows(m0, n0);
    dma(lds0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): step 0 has landed
    __syncthreads();   // for every wave (and the position table is written)
    reads(lds0, 0, fa[0], fb[0]);
    for (int kt = 0; kt < KT; kt += kProjStages) {
      step(lds0, lds1, kt);
      step(lds1, lds0, kt + 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the last loads have landed before LDS is reused
    __syncthreads();

    // ---- epilogue, one half of the tile's tokens at a time (the operand stages are free after the
    // last barrier).  Lane (rr, h) of wave (wm, wn) holds, for token 128 wm + 32 i + rr and packed tile
    // j, the columns 128 wn + 32 j + 8 c + 4 h + r in register 4 c + r.  Half hf takes the token tiles
    // i = 2 hf, 2 hf + 1 of both wm: its 128 tokens go to LDS as fp32 rows of the tile's 256 columns
    // (local row 64 wm + 32 (i - 2 hf) + rr; 16-byte granule g of row r at g ^ (r mod 16)).  Then each
    // token's heads are taken by G = D / 16 adjacent threads, thread k owning the columns
    // [8 k, 8 k + 8) of a head and their rotate-half partners [D/2 + 8 k, D/2 + 8 k + 8): the sum of
    // squares is a reduction over the G lanes, and cos / sin of the thread's 8 pairs serve every head
    // of the token.
    // [128][256] fp32, swizzled granules: rows 64 s + [0, 64) in stage array s
    auto eprow = [&](int lr) {
      uint4* base = lr < 64 ? &lds0[0][0] : &lds1[0][0];
      return reinterpret_cast<float*>(base) + (lr & 63) * kProjBN;
    };
    // the q and k weights of the thread's 16 columns, as fp32 (the same for every token)
    float wqv[16], wkv[16];
  #pragma unroll
    for (int c = 0; c < 8; ++c) {
      wqv[c] = proj_bf16_f32(ep_w[0][8 * k + c]);
      wqv[8 + c] = proj_bf16_f32(ep_w[0][D / 2 + 8 * k + c]);
      wkv[c] = proj_bf16_f32(ep_w[1][8 * k + c]);
      wkv[8 + c] = proj_bf16_f32(ep_w[1][D / 2 + 8 * k + c]);
    }
    const float inv_d = 1.0f / D;
    bool any_qk = false;  // a tile of v heads only needs no angles
#pragma unroll
    for (int hd = 0; hd < HEADS; ++hd) {
      int ty, ix;
      proj_head(a, min(n0 / D + hd, a.heads - 1), ty, ix);
      any_qk |= ty != 2;
    }
  #pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
  #pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * hf + ii, lr = 64 * wm + 32 * ii + rr;
  #pragma unroll
        for (int j = 0; j < 4; ++j)
  #pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int g = 32 * wn + 8 * j + 2 * c + h;
            *reinterpret_cast<float4*>(eprow(lr) + 4 * (g ^ (lr & 15))) =
                make_float4(acc[j][i][4 * c], acc[j][i][4 * c + 1], acc[j][i][4 * c + 2], acc[j][i][4 * c + 3]);
          }
      }
      __syncthreads();
  #pragma unroll
      for (int lr = threadIdx.x / G; lr < 128; lr += TOK_PER_PASS) {  // all passes at once: independent chains
        const int64_t t = m0 + 128 * (lr / 64) + 64 * hf + lr % 64;
        float cs[8], sn[8];
        if (ROPE && any_qk) {
          const int32_t p = ep_pos[128 * (lr / 64) + 64 * hf + lr % 64];
  #pragma unroll
          for (int c = 0; c < 8; ++c) rope_cos_sin(p, ep_turns[8 * k + c], cs[c], sn[c]);
        }
        const float* rowp = eprow(lr);
  #pragma unroll
        for (int hd = 0; hd < HEADS; ++hd) {
          const int hb = (n0 + hd * D) / D;
          int ty, ix;
          proj_head(a, min(hb, a.heads - 1), ty, ix);
          float lo[8], hi[8];
          {
            const int g0 = (hd * D + 8 * k) / 4, g1 = (hd * D + D / 2 + 8 * k) / 4;
            const float4 l0 = *reinterpret_cast<const float4*>(rowp + 4 * (g0 ^ (lr & 15)));
            const float4 l1 = *reinterpret_cast<const float4*>(rowp + 4 * ((g0 + 1) ^ (lr & 15)));
            const float4 h0 = *reinterpret_cast<const float4*>(rowp + 4 * (g1 ^ (lr & 15)));
            const float4 h1 = *reinterpret_cast<const float4*>(rowp + 4 * ((g1 + 1) ^ (lr & 15)));
            lo[0] = l0.x; lo[1] = l0.y; lo[2] = l0.z; lo[3] = l0.w; lo[4] = l1.x; lo[5] = l1.y; lo[6] = l1.z; lo[7] = l1.w;
            hi[0] = h0.x; hi[1] = h0.y; hi[2] = h0.z; hi[3] = h0.w; hi[4] = h1.x; hi[5] = h1.y; hi[6] = h1.z; hi[7] = h1.w;
          }
          if (ty != 2) {
            float ssq = 0.0f;
  #pragma unroll
            for (int c = 0; c < 8; ++c) ssq = fmaf(lo[c], lo[c], fmaf(hi[c], hi[c], ssq));
            ssq = proj_group_sum<G>(ssq);
            const float r = rsqrtf(fmaf(ssq, inv_d, a.eps));
            const float* wv = ty == 0 ? wqv : wkv;
  #pragma unroll
            for (int c = 0; c < 8; ++c) {
              const float nl = lo[c] * r * wv[c], nh = hi[c] * r * wv[8 + c];
              if constexpr (ROPE) {
                lo[c] = nl * cs[c] - nh * sn[c];
                hi[c] = nh * cs[c] + nl * sn[c];
              } else {
                lo[c] = nl;
                hi[c] = nh;
              }
            }
          }
          if (t < a.T && hb < a.heads) {
            uint16_t* base = ty == 0 ? a.q : (ty == 1 ? a.k : a.v);
            const int nh = ty == 0 ? a.n_q : a.n_kv;
            uint16_t* dst = base + (t * nh + ix) * D + 8 * k;
            st16(dst, make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(lo[4], lo[5]),
                                 pack_bf16x2(lo[6], lo[7])));
            st16(dst + D / 2, make_uint4(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]),
                                         pack_bf16x2(hi[4], hi[5]), pack_bf16x2(hi[6], hi[7])));
          }
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace qkvnr
