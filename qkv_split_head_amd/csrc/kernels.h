// gfx950 kernels of the packed-QKV split + per-head RMSNorm + RoPE path.
//
// Work decomposition.  The packed row of one token is a sequence of `heads`
// head blocks of D values (n_q + 2 n_kv blocks; the layout decides which block
// is which head).  A wave walks a token's row in iterations of HPI whole heads
// (64 lanes x 16 bytes = 1 KiB per load instruction, fully coalesced); a work
// unit is one token's row, or a segment of it when there are too few tokens to
// fill the chip.  Units are handed out grid-stride to waves.  Each unit reads
// its position once and computes cos/sin once: lane L evaluates pair frequency
// L mod R/2, and each lane gathers the EPC frequencies of its chunk with
// ds_bpermute; the same values serve every head of the token.
//
// Arithmetic per head (fp32): ss = sum x^2 over the head's lanes (DPP, no
// LDS), r = 1/sqrt(ss/D + eps), n = x r w, y = n cos + (+/-) partner(n) sin,
// one rounding at the store.  v heads are stored as the loaded bits.
#pragma once

#include "device.h"

namespace qkvnr {

constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWave * kWavesPerBlock;
constexpr int kUnroll = 4;  // wave iterations whose loads are issued together

enum : int { kInterleaved = 0, kSectioned = 1 };

struct GqaArgs {
  const uint8_t* qkv;  // packed input
  int64_t row_bytes;   // bytes between tokens of qkv (and of dqkv)
  const int32_t* pos;
  const uint8_t* wq;
  const uint8_t* wk;
  // forward outputs (k/v are pools [pages, page_size, n_kv, D] when paged)
  uint8_t* q;
  uint8_t* k;
  uint8_t* v;
  // backward
  const uint8_t* dq;
  const uint8_t* dk;
  const uint8_t* dv;
  uint8_t* dqkv;
  float* dwq;
  float* dwk;
  float eps;
  float inv_d;
  double log2_theta;
  int32_t kind;
  int32_t n_kv;
  int32_t q_per_kv;
  int32_t n_q;
  int32_t heads;      // head blocks per token
  int32_t iters;      // wave iterations per token
  int32_t seg_iters;  // wave iterations per work unit
  int32_t nseg;       // work units per token
  int64_t units;      // T * nseg
  uint32_t grp_magic; // ceil(2^32 / (q_per_kv + 2)), exact division for head < 2^16
  // paged store
  const int32_t* bt;
  int32_t bt_stride;
  int32_t tokens_per_req;
  int32_t page_size;
  int32_t num_pages;
};

// Which output head a packed head block is: type 0 = q, 1 = k, 2 = v, and its index.
__device__ __forceinline__ void map_head(const GqaArgs& a, int h, int& type, int& idx) {
  if (a.kind == kInterleaved) {
    const int g = static_cast<int>(__umulhi(static_cast<uint32_t>(h), a.grp_magic));
    const int s = h - g * (a.q_per_kv + 2);
    type = s < a.q_per_kv ? 0 : (s == a.q_per_kv ? 1 : 2);
    idx = type == 0 ? g * a.q_per_kv + s : g;
  } else {
    type = h < a.n_q ? 0 : (h < a.n_q + a.n_kv ? 1 : 2);
    idx = h - (type == 0 ? 0 : (type == 1 ? a.n_q : a.n_q + a.n_kv));
  }
}

// cos/sin for the EPC pair frequencies of this lane's chunk at position p.
// `tpp` is lane L's turns-per-position for frequency L mod R/2.  The sine is
// returned with the rotate-half sign folded in: -sin for the first half of the
// head (y_i = n_i cos - n_{i+R/2} sin), +sin for the second half.
template <int EPC, int LPH>
__device__ __forceinline__ void unit_cos_sin(int32_t p, double tpp, int c, float (&cs)[EPC],
                                             float (&sn)[EPC]) {
  float cv, sv;
  rope_cos_sin(p, tpp, cv, sv);
  const int fbase = (c % (LPH / 2)) * EPC;
  const float sgn = c < LPH / 2 ? -1.0f : 1.0f;
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    cs[e] = __shfl(cv, fbase + e, kWave);
    sn[e] = sgn * __shfl(sv, fbase + e, kWave);
  }
}

// Pool slot of token t (paged store), or -1 when the table does not map it.
__device__ __forceinline__ int64_t paged_slot(const int32_t* bt, int32_t bt_stride,
                                              int32_t tokens_per_req, int32_t page_size,
                                              int32_t num_pages, int64_t t, int32_t p) {
  if (p < 0) return -1;
  const int32_t pi = p / page_size;
  if (pi >= bt_stride) return -1;
  const int64_t b = t / tokens_per_req;
  const int32_t page = bt[b * bt_stride + pi];
  if (page < 0 || page >= num_pages) return -1;
  return static_cast<int64_t>(page) * page_size + (p - pi * page_size);
}

// ------------------------------------------------------------------ forward

template <typename IO, int D, bool ROPE, bool PAGED>
__global__ __launch_bounds__(kBlockThreads) void fwd_gqa_kernel(const GqaArgs a) {
  constexpr int EPC = Chunk<IO>::EPC;
  constexpr int LPH = D / EPC;
  constexpr int HPI = kWave / LPH;
  constexpr int HB = D * static_cast<int>(sizeof(IO));  // bytes per head
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & (LPH - 1);
  const int hs = lane / LPH;
  const int c = chunk_of_lane<LPH>(li);
  const int cb = c * 16;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;

  float wq[EPC], wk[EPC];
  unpack(ld16(a.wq + cb), wq);
  unpack(ld16(a.wk + cb), wk);
  double tpp = 0.0;
  if constexpr (ROPE) tpp = turns_per_position(lane % (D / 2), D, a.log2_theta);

  for (int64_t u = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; u < a.units; u += nwaves) {
    const int64_t t = a.nseg == 1 ? u : u / a.nseg;
    const int sg = static_cast<int>(u - t * a.nseg);
    const int it0 = sg * a.seg_iters;
    const int it1 = min(it0 + a.seg_iters, a.iters);

    int32_t p = 0;
    if constexpr (ROPE || PAGED) p = a.pos[t];
    float cs[EPC], sn[EPC];
    if constexpr (ROPE) unit_cos_sin<EPC, LPH>(p, tpp, c, cs, sn);
    int64_t kv_tok = t;
    if constexpr (PAGED) kv_tok = paged_slot(a.bt, a.bt_stride, a.tokens_per_req, a.page_size, a.num_pages, t, p);

    const uint8_t* row = a.qkv + t * a.row_bytes;
    for (int it = it0; it < it1; it += kUnroll) {
      uint4 buf[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int h = (it + j) * HPI + hs;
        buf[j] = make_uint4(0u, 0u, 0u, 0u);
        if (it + j < it1 && h < a.heads) buf[j] = ld16(row + h * HB + cb);
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        if (it + j >= it1) break;  // wave-uniform
        const int h = (it + j) * HPI + hs;
        int type, idx;
        map_head(a, h, type, idx);
        float x[EPC];
        unpack(buf[j], x);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) ss = fmaf(x[e], x[e], ss);
        ss = head_sum<LPH>(ss);
        const float r = rsqrtf(ss * a.inv_d + a.eps);
        float y[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) y[e] = x[e] * r * (type == 0 ? wq[e] : wk[e]);
        if constexpr (ROPE) {
          float z[EPC];
#pragma unroll
          for (int e = 0; e < EPC; ++e) z[e] = fmaf(y[e], cs[e], partner<LPH>(y[e]) * sn[e]);
#pragma unroll
          for (int e = 0; e < EPC; ++e) y[e] = z[e];
        }
        const uint4 out = type == 2 ? buf[j] : pack(y);
        if (h < a.heads) {
          if (type == 0) {
            st16(a.q + (t * a.n_q + idx) * HB + cb, out);
          } else if (kv_tok >= 0) {
            st16((type == 1 ? a.k : a.v) + (kv_tok * a.n_kv + idx) * HB + cb, out);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ backward

// dwq/dwk must be zero before the launch; each block adds its partial sums.
template <typename IO, int D, bool ROPE>
__global__ __launch_bounds__(kBlockThreads) void bwd_gqa_kernel(const GqaArgs a) {
  constexpr int EPC = Chunk<IO>::EPC;
  constexpr int LPH = D / EPC;
  constexpr int HPI = kWave / LPH;
  constexpr int HB = D * static_cast<int>(sizeof(IO));
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & (LPH - 1);
  const int hs = lane / LPH;
  const int c = chunk_of_lane<LPH>(li);
  const int cb = c * 16;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;

  float wq[EPC], wk[EPC];
  unpack(ld16(a.wq + cb), wq);
  unpack(ld16(a.wk + cb), wk);
  double tpp = 0.0;
  if constexpr (ROPE) tpp = turns_per_position(lane % (D / 2), D, a.log2_theta);
  float accq[EPC], acck[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) accq[e] = acck[e] = 0.0f;

  for (int64_t u = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; u < a.units; u += nwaves) {
    const int64_t t = a.nseg == 1 ? u : u / a.nseg;
    const int sg = static_cast<int>(u - t * a.nseg);
    const int it0 = sg * a.seg_iters;
    const int it1 = min(it0 + a.seg_iters, a.iters);
    float cs[EPC], sn[EPC];
    if constexpr (ROPE) unit_cos_sin<EPC, LPH>(a.pos[t], tpp, c, cs, sn);
    const uint8_t* row = a.qkv + t * a.row_bytes;
    uint8_t* drow = a.dqkv + t * a.row_bytes;

    for (int it = it0; it < it1; it += kUnroll) {
      uint4 xb[kUnroll], gb[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int h = (it + j) * HPI + hs;
        xb[j] = gb[j] = make_uint4(0u, 0u, 0u, 0u);
        if (it + j < it1 && h < a.heads) {
          int type, idx;
          map_head(a, h, type, idx);
          const uint8_t* g = type == 0 ? a.dq + (t * a.n_q + idx) * HB
                                       : (type == 1 ? a.dk : a.dv) + (t * a.n_kv + idx) * HB;
          gb[j] = ld16(g + cb);
          if (type != 2) xb[j] = ld16(row + h * HB + cb);
        }
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        if (it + j >= it1) break;  // wave-uniform
        const int h = (it + j) * HPI + hs;
        const bool valid = h < a.heads;
        int type, idx;
        map_head(a, h, type, idx);
        float x[EPC], g[EPC];
        unpack(xb[j], x);
        unpack(gb[j], g);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) ss = fmaf(x[e], x[e], ss);
        ss = head_sum<LPH>(ss);
        const float r = rsqrtf(ss * a.inv_d + a.eps);
        float uu[EPC];
        if constexpr (ROPE) {
          // transpose of the forward rotation: u = g cos - partner(g) * (signed sin)
#pragma unroll
          for (int e = 0; e < EPC; ++e) uu[e] = fmaf(g[e], cs[e], -partner<LPH>(g[e]) * sn[e]);
        } else {
#pragma unroll
          for (int e = 0; e < EPC; ++e) uu[e] = g[e];
        }
        float xh[EPC], av[EPC];
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          xh[e] = x[e] * r;
          av[e] = uu[e] * (type == 0 ? wq[e] : wk[e]);
          dot = fmaf(av[e], xh[e], dot);
        }
        dot = head_sum<LPH>(dot);
        const float m = dot * a.inv_d;
        float dx[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) dx[e] = r * fmaf(-xh[e], m, av[e]);
        if (valid) {
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            const float term = uu[e] * xh[e];
            if (type == 0) accq[e] += term;
            else if (type == 1) acck[e] += term;
          }
          st16(drow + h * HB + cb, type == 2 ? gb[j] : pack(dx));
        }
      }
    }
  }

  // norm-weight grads: lanes holding the same chunk (same li) -> lanes 0..LPH-1,
  // then the block's waves through LDS, then one atomic add per value per block.
#pragma unroll
  for (int off = LPH; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      accq[e] += __shfl_xor(accq[e], off, kWave);
      acck[e] += __shfl_xor(acck[e], off, kWave);
    }
  }
  __shared__ float red[kWavesPerBlock][2][D];
  if (hs == 0) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      red[wave][0][c * EPC + e] = accq[e];
      red[wave][1][c * EPC + e] = acck[e];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * D; i += kBlockThreads) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) s += red[w][i / D][i % D];
    atomicAdd(i < D ? a.dwq + i : a.dwk + (i - D), s);
  }
}

__global__ void zero2_f32_kernel(float* a, float* b, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    a[i] = 0.0f;
    b[i] = 0.0f;
  }
}

// ------------------------------------------------------------------ latent rows

struct LatentArgs {
  const uint8_t* rows;
  int64_t row_bytes;
  const int32_t* pos;
  const uint8_t* w;
  uint8_t* out;  // [T, 576] or pool [pages, page_size, 576]
  float eps;
  double log2_theta;
  int64_t T;
  const int32_t* bt;
  int32_t bt_stride;
  int32_t tokens_per_req;
  int32_t page_size;
  int32_t num_pages;
};

// bf16 rows of 512 normed values (one 16-byte chunk per lane) and 64 rotated
// values (8 lanes, mirror chunk order); one wave per row.
template <bool PAGED>
__global__ __launch_bounds__(kBlockThreads) void fwd_latent_kernel(const LatentArgs a) {
  constexpr int NORM = 512, ROPE_D = 64, ROW_B = (NORM + ROPE_D) * 2, NORM_B = NORM * 2;
  constexpr int LPR = 8;  // lanes of the rotated tail
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & (LPR - 1);
  const int c = chunk_of_lane<LPR>(li);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  float w[8];
  unpack(ld16(a.w + lane * 16), w);
  const double tpp = turns_per_position(lane % (ROPE_D / 2), ROPE_D, a.log2_theta);

  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; t < a.T; t += nwaves) {
    const uint8_t* row = a.rows + t * a.row_bytes;
    const uint4 xn = ld16(row + lane * 16);
    uint4 xr = make_uint4(0u, 0u, 0u, 0u);
    if (lane < LPR) xr = ld16(row + NORM_B + c * 16);
    const int32_t p = a.pos[t];
    float cs[8], sn[8];
    unit_cos_sin<8, LPR>(p, tpp, c, cs, sn);

    float x[8];
    unpack(xn, x);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss = head_sum<kWave>(ss);
    const float r = rsqrtf(ss * (1.0f / NORM) + a.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * r * w[e];

    float k[8], z[8];
    unpack(xr, k);
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = fmaf(k[e], cs[e], partner<LPR>(k[e]) * sn[e]);

    int64_t dst = t;
    if constexpr (PAGED) dst = paged_slot(a.bt, a.bt_stride, a.tokens_per_req, a.page_size, a.num_pages, t, p);
    if (dst >= 0) {
      uint8_t* o = a.out + dst * ROW_B;
      st16(o + lane * 16, pack(x));
      if (lane < LPR) st16(o + NORM_B + c * 16, pack(z));
    }
  }
}

}  // namespace qkvnr
