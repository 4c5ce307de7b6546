// gfx950 kernels of the packed-QKV split + per-head RMSNorm + RoPE path.
//
// Work decomposition.  The packed row of one token is a sequence of `heads`
// head blocks of D values (n_q + 2 n_kv blocks; the layout decides which block
// is which head).  A wave iteration covers HPI whole heads: 64 lanes x 16 bytes
// = 1 KiB per load instruction, fully coalesced.  A token's row takes `iters`
// iterations; a work unit is U consecutive iterations of one token, and each
// wave does exactly one unit: it issues all of its loads at once, computes the
// token's cos/sin while they are in flight, then normalises, rotates, stores
// and exits.  Short-lived waves keep the memory pipeline full: on gfx9-class
// hardware one counter tracks loads and stores in issue order, so a wave that
// looped would wait for its own earlier stores before each new batch of loads.
//
// cos/sin: lane L evaluates pair frequency L mod R/2 at the token's position
// (angle formed in fp64, frequencies tabled on the host) and each lane gathers
// the EPC frequencies of its chunk with ds_bpermute.
//
// Arithmetic per head (fp32): ss = sum x^2 over the head's lanes (DPP, no
// LDS), r = 1/sqrt(ss/D + eps), n = x r w, y = n cos + (+/-) partner(n) sin,
// one rounding at the store.  v heads are stored as the loaded bits.
#pragma once

#include "device.h"

#ifndef QKVNR_FWD_UNITS
#define QKVNR_FWD_UNITS 4
#endif
#ifndef QKVNR_FWD_DEPTH
#define QKVNR_FWD_DEPTH 3
#endif
#ifndef QKVNR_BWD_UNITS
#define QKVNR_BWD_UNITS 4
#endif
#ifndef QKVNR_BWD_DEPTH
#define QKVNR_BWD_DEPTH QKVNR_BWD_UNITS
#endif
#ifndef QKVNR_NT_LOADS
#define QKVNR_NT_LOADS 1
#endif
#ifndef QKVNR_NT_STORES
#define QKVNR_NT_STORES 1
#endif

namespace qkvnr {

#ifndef QKVNR_BWD_WAVES_PER_BLOCK
#define QKVNR_BWD_WAVES_PER_BLOCK 4
#endif

constexpr int kWavesPerBlock = 4;  // forward and latent kernels
constexpr int kBlockThreads = kWave * kWavesPerBlock;
// backward: larger blocks mean fewer block partial sums of the weight grads
constexpr int kBwdWavesPerBlock = QKVNR_BWD_WAVES_PER_BLOCK;
constexpr int kBwdBlockThreads = kWave * kBwdWavesPerBlock;
constexpr int kFwdU = QKVNR_FWD_UNITS;  // wave iterations per forward work unit
constexpr int kFwdDepth = QKVNR_FWD_DEPTH;  // forward streaming loads in flight per wave
constexpr int kBwdU = QKVNR_BWD_UNITS;  // wave iterations per backward work unit
constexpr int kBwdDepth = QKVNR_BWD_DEPTH;  // backward iterations whose loads are in flight per wave
static_assert(kFwdDepth >= 1 && kFwdDepth <= kFwdU, "forward load depth must be in [1, units]");
static_assert(kBwdDepth >= 1 && kBwdDepth <= kBwdU, "backward load depth must be in [1, units]");
constexpr int kMaxPairs = 64;           // rotate-half pairs of the widest rotated head (D = 128)
constexpr int kWgradSlots = 16;         // backward weight-grad partial-sum slots

enum : int { kInterleaved = 0, kSectioned = 1 };

__device__ __forceinline__ uint4 ld_stream(const void* p) {
  if constexpr (QKVNR_NT_LOADS) return ld16_nt(p);
  else return ld16(p);
}
__device__ __forceinline__ void st_stream(void* p, const uint4& v) {
  if constexpr (QKVNR_NT_STORES) st16_nt(p, v);
  else st16(p, v);
}

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
  float* slots;         // [kWgradSlots][2 * D] partial sums, zero between calls
  float eps;
  float inv_d;
  int64_t T;
  int64_t units;        // T * units_per_token
  int64_t unit0;        // first work unit of this launch (a large batch takes several launches)
  uint64_t upt_magic;   // ceil(2^64 / upt) for upt > 1: unit / upt = umul64hi(unit, magic)
  int32_t upt;          // work units per token
  int32_t kind;
  int32_t n_kv;
  int32_t q_per_kv;
  int32_t n_q;
  int32_t heads;        // head blocks per token
  int32_t iters;        // wave iterations per token
  uint32_t q_magic;     // ceil(2^32 / q_per_kv), exact division for head < 2^16
  // paged store
  const int32_t* bt;
  int32_t bt_stride;
  int32_t tokens_per_req;
  int32_t page_size;
  int32_t num_pages;
  // turns per position of rotate-half pair i: theta^(-2i/R) / (2 pi)
  double turns[kMaxPairs];
};

// Heads are taken kind-major in both layouts: head h < n_q is q head h, then come the n_kv k heads and the
// n_kv v heads.  So every iteration of HPI heads is one kind when n_q and n_kv are multiples of HPI (the
// interleaved Muse layout as much as the sectioned one), and iter_kind's uniform bodies apply.
// type 0 = q, 1 = k, 2 = v, and the head's index in its output.
__device__ __forceinline__ void map_head(const GqaArgs& a, int h, int& type, int& idx) {
  type = h < a.n_q ? 0 : (h < a.n_q + a.n_kv ? 1 : 2);
  idx = h - (type == 0 ? 0 : (type == 1 ? a.n_q : a.n_q + a.n_kv));
}

// Where head h sits in the packed row, in head blocks: h itself in the sectioned layout; in the interleaved
// one q head g Q + s is block g (Q + 2) + s, and the k and v heads of group g are blocks g (Q + 2) + Q and
// g (Q + 2) + Q + 1.  An iteration's blocks are then not one span of the row (HPI q heads span 1 + HPI / Q
// groups, HPI k heads sit one group apart), but each block is whole 128-byte lines.
template <bool ILV>
__device__ __forceinline__ int mem_head(const GqaArgs& a, int h) {
  if constexpr (!ILV) {
    return h;
  } else {
    const int Q = a.q_per_kv;
    if (h < a.n_q) {
      const int g = static_cast<int>(__umulhi(static_cast<uint32_t>(h), a.q_magic));
      return g * (Q + 2) + (h - g * Q);
    }
    return h < a.n_q + a.n_kv ? (h - a.n_q) * (Q + 2) + Q : (h - a.n_q - a.n_kv) * (Q + 2) + Q + 1;
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

// What the heads of one wave iteration are, decided once for the wave: all q
// (0), all k (1), all v (2), or a mix (3).  A uniform iteration takes a body
// compiled for its one head type: one weight, one output, no per-lane selects,
// and a v iteration does no arithmetic at all.  Lane 0 always holds a head of
// the row; lanes past the last head do not count.
enum : int { kAllQ = 0, kAllK = 1, kAllV = 2, kMixed = 3 };
__device__ __forceinline__ int iter_kind(int h, int heads, int type) {
  const int first = __builtin_amdgcn_readfirstlane(type);
  return __builtin_amdgcn_ballot_w64(h < heads && type != first) == 0 ? first : kMixed;
}

template <typename IO, int D>
struct Geo {
  static constexpr int EPC = Chunk<IO>::EPC;
  static constexpr int LPH = D / EPC;                          // lanes per head
  static constexpr int HPI = kWave / LPH;                      // heads per wave iteration
  static constexpr int HB = D * static_cast<int>(sizeof(IO));  // bytes per head
};

// This wave's work unit: token t and its first iteration it0 (wave-uniform).
__device__ __forceinline__ bool wave_unit(const GqaArgs& a, int U, int waves_per_block, int64_t& t, int& it0) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int64_t unit = a.unit0 + static_cast<int64_t>(blockIdx.x) * waves_per_block + wave;
  if (unit >= a.units) return false;
  t = a.upt == 1 ? unit  // one unit per token: no division (and no 2^64 magic)
                 : static_cast<int64_t>(__umul64hi(static_cast<uint64_t>(unit), a.upt_magic));
  it0 = static_cast<int>(unit - t * a.upt) * U;
  return true;
}

// ------------------------------------------------------------------ forward

// One forward iteration of the lane's head h (type, idx from map_head; kind
// from iter_kind): normalise, rotate, round once and store to q, k or v (a v
// head stores the loaded bits).  kv_tok is the token's k/v row (its pool slot
// when paged, -1 when the table does not map it).
template <typename IO, int D, bool ROPE>
__device__ __forceinline__ void fwd_iter(int kind, const uint4& xb, const uint4& wq_raw, const uint4& wk_raw,
                                         const float (&cs)[Geo<IO, D>::EPC], const float (&sn)[Geo<IO, D>::EPC],
                                         float eps, float inv_d, int h, int heads, int type, int idx, int cb,
                                         uint8_t* q, uint8_t* k, uint8_t* v, int64_t t, int64_t kv_tok, int n_q,
                                         int n_kv) {
  using G = Geo<IO, D>;
  constexpr int EPC = G::EPC, LPH = G::LPH, HB = G::HB;
  if (kind == kAllV) {  // wave-uniform: a copy, no arithmetic
    if (h < heads && kv_tok >= 0) st_stream(v + (kv_tok * n_kv + idx) * HB + cb, xb);
    return;
  }
  float x[EPC];
  unpack(xb, x);
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < EPC; ++e) ss = fmaf(x[e], x[e], ss);
  ss = head_sum<LPH>(ss);
  const float r = rsqrtf(ss * inv_d + eps);
  float w[EPC], y[EPC];
  unpack(type == 0 ? wq_raw : wk_raw, w);
#pragma unroll
  for (int e = 0; e < EPC; ++e) y[e] = x[e] * r * w[e];
  if constexpr (ROPE) {
    float z[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) z[e] = fmaf(y[e], cs[e], partner<LPH>(y[e]) * sn[e]);
#pragma unroll
    for (int e = 0; e < EPC; ++e) y[e] = z[e];
  }
  if (kind == kAllQ) {  // wave-uniform branches: one output, no per-lane selects
    if (h < heads) st_stream(q + (t * n_q + idx) * HB + cb, pack(y));
  } else if (kind == kAllK) {
    if (h < heads && kv_tok >= 0) st_stream(k + (kv_tok * n_kv + idx) * HB + cb, pack(y));
  } else {
    const uint4 out = type == 2 ? xb : pack(y);
    uint8_t* dst = type == 0 ? q + (t * n_q + idx) * HB : (type == 1 ? k : v) + (kv_tok * n_kv + idx) * HB;
    if (h < heads && (type == 0 || kv_tok >= 0)) st_stream(dst + cb, out);
  }
}

// U iterations per work unit, DEPTH of their loads in flight at once: (kFwdU,
// kFwdDepth) for streaming batches, (1, 1) for small batches, where the
// shortest per-wave chain (one load, one store) gives the lowest latency.
template <typename IO, int D, bool ROPE, bool PAGED, int U, int DEPTH, bool ILV>
__global__ __launch_bounds__(kBlockThreads) void fwd_gqa_kernel(const GqaArgs a) {
  static_assert(DEPTH >= 1 && DEPTH <= U, "load depth must be in [1, units]");
  using G = Geo<IO, D>;
  constexpr int EPC = G::EPC, LPH = G::LPH, HPI = G::HPI, HB = G::HB;
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & (LPH - 1);
  const int hs = lane / LPH;
  const int c = chunk_of_lane<LPH>(li);
  const int cb = c * 16;

  int64_t t;
  int it0;
  if (!wave_unit(a, U, kWavesPerBlock, t, it0)) return;
  const int n_it = min(U, a.iters - it0);

  // Small operands first: the vector memory counter completes in issue order,
  // so loads issued before the streaming loads can be waited for alone.
  // This lane's chunk of each norm weight stays packed until a head picks one.
  const uint4 wq_raw = ld16(a.wq + cb), wk_raw = ld16(a.wk + cb);
  double tpp = 0.0;
  if constexpr (ROPE) tpp = a.turns[lane % (D / 2)];
  int32_t p = 0;
  if constexpr (ROPE || PAGED) p = a.pos[t];  // t is wave-uniform: a scalar load
  int64_t kv_tok = t;
  if constexpr (PAGED) kv_tok = paged_slot(a.bt, a.bt_stride, a.tokens_per_req, a.page_size, a.num_pages, t, p);
  __builtin_amdgcn_sched_barrier(0);

  // Streaming loads without branches: a lane past the last head re-reads the
  // last head block (same row, already in flight), and its result is dropped.
  // DEPTH of them go out at once; each store is followed by the next load.
  const uint8_t* row = a.qkv + t * a.row_bytes;
  uint4 buf[U];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j)
    buf[j] = ld_stream(row + mem_head<ILV>(a, min((it0 + j) * HPI + hs, a.heads - 1)) * HB + cb);
  __builtin_amdgcn_sched_barrier(0);

  float cs[EPC], sn[EPC];
  if constexpr (ROPE) unit_cos_sin<EPC, LPH>(p, tpp, c, cs, sn);

#pragma unroll
  for (int j = 0; j < U; ++j) {
    if (j >= n_it) break;  // wave-uniform
    const int h = (it0 + j) * HPI + hs;
    int type, idx;
    map_head(a, h, type, idx);
    fwd_iter<IO, D, ROPE>(iter_kind(h, a.heads, type), buf[j], wq_raw, wk_raw, cs, sn, a.eps, a.inv_d, h, a.heads,
                          type, idx, cb, a.q, a.k, a.v, t, kv_tok, a.n_q, a.n_kv);
    if (j + DEPTH < U) {
      __builtin_amdgcn_sched_barrier(0);
      buf[j + DEPTH] = ld_stream(row + mem_head<ILV>(a, min((it0 + j + DEPTH) * HPI + hs, a.heads - 1)) * HB + cb);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ------------------------------------------------------------------ backward

// Weight grads: per lane over the unit, then the wave (shuffles), then the
// block (LDS), then one fp32 atomic per value into slot (block mod 16) of the
// workspace; wgrad_fold_kernel then sums the slots.  Atomics on one address
// serialise (tens of ns each), so the slot count trades that contention
// against the fold's reads: with 16 slots a slot's address takes a fifth of
// the kernel's time in atomics, with 4 most of it.  A single-launch hand-over (the last
// block to finish folds) would need every block to wait for returning atomics
// or to fence, which costs more than the second launch on a multi-XCD part.
// One iteration's backward loads for the lane's head block h: its output
// cotangent and, for q/k heads, its input.  Lanes past the last head re-read
// the last head, and a v head, whose input is not needed, reads the q weight
// chunk (cached) in place of its input chunk: no load is skipped, because a
// skipped load would turn every later wait into a full drain.
template <int HB, bool ILV>
// (`a` by value: with a reference to the kernel argument block the compiler
// copies the whole block to scratch.)
__device__ __forceinline__ void bwd_load(const GqaArgs a, int64_t t, int h, const uint8_t* row, int cb,
                                         uint4& xb, uint4& gb) {
  h = min(h, a.heads - 1);
  int type, idx;
  map_head(a, h, type, idx);
  const uint8_t* g = type == 0 ? a.dq + (t * a.n_q + idx) * HB
                               : (type == 1 ? a.dk : a.dv) + (t * a.n_kv + idx) * HB;
  gb = ld_stream(g + cb);
  xb = ld_stream(type != 2 ? row + mem_head<ILV>(a, h) * HB + cb : a.wq + cb);
}

// One backward iteration of the lane's head h (type from map_head; kind from
// iter_kind): the cotangent rotated back, the RMSNorm backward recomputed from
// the packed input, the packed grad stored in dqkv (a v head stores the loaded
// cotangent bits) and the head's weight-grad terms u x^ added to the lane's sums.
template <typename IO, int D, bool ROPE>
__device__ __forceinline__ void bwd_iter(int kind, const uint4& xb, const uint4& gb, const uint4& wq_raw,
                                         const uint4& wk_raw, const float (&cs)[Geo<IO, D>::EPC],
                                         const float (&sn)[Geo<IO, D>::EPC], float eps, float inv_d, int h, int heads,
                                         int type, uint8_t* drow, int cb, float (&accq)[Geo<IO, D>::EPC],
                                         float (&acck)[Geo<IO, D>::EPC]) {
  using G = Geo<IO, D>;
  constexpr int EPC = G::EPC, LPH = G::LPH, HB = G::HB;
  if (kind == kAllV) {  // wave-uniform: the cotangent is the grad, no arithmetic
    if (h < heads) st_stream(drow + h * HB + cb, gb);
    return;
  }
  float x[EPC], g[EPC];
  unpack(xb, x);
  unpack(gb, g);
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < EPC; ++e) ss = fmaf(x[e], x[e], ss);
  ss = head_sum<LPH>(ss);
  const float r = rsqrtf(ss * inv_d + eps);
  float uu[EPC];
  if constexpr (ROPE) {
    // transpose of the forward rotation: u = g cos - partner(g) * (signed sin)
#pragma unroll
    for (int e = 0; e < EPC; ++e) uu[e] = fmaf(g[e], cs[e], -partner<LPH>(g[e]) * sn[e]);
  } else {
#pragma unroll
    for (int e = 0; e < EPC; ++e) uu[e] = g[e];
  }
  float w[EPC], xh[EPC], av[EPC];
  unpack(type == 0 ? wq_raw : wk_raw, w);
  float dot = 0.0f;
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    xh[e] = x[e] * r;
    av[e] = uu[e] * w[e];
    dot = fmaf(av[e], xh[e], dot);
  }
  dot = head_sum<LPH>(dot);
  const float m = dot * inv_d;
  float dx[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) dx[e] = r * fmaf(-xh[e], m, av[e]);
  if (h < heads) {
    if (kind == kAllQ) {  // wave-uniform branches: one sum, no per-lane selects
#pragma unroll
      for (int e = 0; e < EPC; ++e) accq[e] = fmaf(uu[e], xh[e], accq[e]);
      st_stream(drow + h * HB + cb, pack(dx));
    } else if (kind == kAllK) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) acck[e] = fmaf(uu[e], xh[e], acck[e]);
      st_stream(drow + h * HB + cb, pack(dx));
    } else {
      // value selects, not a choice of array (that would move both
      // accumulators to scratch); a select also keeps a v head's unused
      // term (NaN when eps = 0) out of the sums
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float term = uu[e] * xh[e];
        accq[e] += type == 0 ? term : 0.0f;
        acck[e] += type == 1 ? term : 0.0f;
      }
      st_stream(drow + h * HB + cb, type == 2 ? gb : pack(dx));
    }
  }
}

template <typename IO, int D, bool ROPE, bool ILV>
__global__ __launch_bounds__(kBwdBlockThreads) void bwd_gqa_kernel(const GqaArgs a) {
  using G = Geo<IO, D>;
  constexpr int EPC = G::EPC, LPH = G::LPH, HPI = G::HPI, HB = G::HB, U = kBwdU;
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & (LPH - 1);
  const int hs = lane / LPH;
  const int c = chunk_of_lane<LPH>(li);
  const int cb = c * 16;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);

  float accq[EPC], acck[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) accq[e] = acck[e] = 0.0f;

  int64_t t;
  int it0;
  if (wave_unit(a, U, kBwdWavesPerBlock, t, it0)) {  // wave-uniform; every wave reaches the block reduction
    const int n_it = min(U, a.iters - it0);
    // small operands first (see the forward kernel)
    const uint4 wq_raw = ld16(a.wq + cb), wk_raw = ld16(a.wk + cb);
    double tpp = 0.0;
    int32_t p = 0;
    if constexpr (ROPE) {
      tpp = a.turns[lane % (D / 2)];
      p = a.pos[t];
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* row = a.qkv + t * a.row_bytes;
    uint4 xb[U], gb[U];
    // kBwdDepth iterations' loads go out at once; each store is followed by
    // the loads of the next iteration
#pragma unroll
    for (int j = 0; j < kBwdDepth; ++j) bwd_load<HB, ILV>(a, t, (it0 + j) * HPI + hs, row, cb, xb[j], gb[j]);
    __builtin_amdgcn_sched_barrier(0);
    float cs[EPC], sn[EPC];
    if constexpr (ROPE) unit_cos_sin<EPC, LPH>(p, tpp, c, cs, sn);

    uint8_t* drow = a.dqkv + t * a.row_bytes;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (j >= n_it) break;  // wave-uniform
      const int h = (it0 + j) * HPI + hs;
      int type, idx;
      map_head(a, h, type, idx);
      // bwd_iter stores head h at drow + h HB: in the interleaved layout the row pointer is shifted so that
      // this lands on the head's block (the sectioned layout passes the row itself)
      uint8_t* dr = drow;
      if constexpr (ILV) dr += static_cast<int64_t>(mem_head<ILV>(a, h) - h) * HB;
      bwd_iter<IO, D, ROPE>(iter_kind(h, a.heads, type), xb[j], gb[j], wq_raw, wk_raw, cs, sn, a.eps, a.inv_d, h,
                            a.heads, type, dr, cb, accq, acck);
      if (j + kBwdDepth < U) {
        __builtin_amdgcn_sched_barrier(0);
        bwd_load<HB, ILV>(a, t, (it0 + j + kBwdDepth) * HPI + hs, row, cb, xb[j + kBwdDepth], gb[j + kBwdDepth]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Every lane's sums go to LDS as they are (contiguous EPC values per lane,
  // 16-byte writes): no cross-lane shuffles, which would cost a chain of
  // LDS-crossbar permutes per value.  After the barrier each value's sum runs
  // over the block's waves and each wave's HPI head slots.
  __shared__ float red[kBwdWavesPerBlock * HPI][2][D];
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    red[wave * HPI + hs][0][c * EPC + e] = accq[e];
    red[wave * HPI + hs][1][c * EPC + e] = acck[e];
  }
  // a barrier that orders LDS only: __syncthreads() would also make every
  // wave wait for its streaming stores to be acknowledged first
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  float* slot = a.slots + (blockIdx.x % kWgradSlots) * (2 * D);
  for (int i = threadIdx.x; i < 2 * D; i += kBwdBlockThreads) {
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kBwdWavesPerBlock * HPI; ++k) s += red[k][i / D][i % D];
    atomicAdd(slot + i, s);
  }
}

// Folds the slots into dq_norm_w / dk_norm_w and zeroes them for the next
// call.  Launched right after the backward on the same stream, so the kernel
// boundary orders it after every block's atomics.  One block of kFoldThreads:
// thread (q, i) sums slots q, q + Q, ... of value i (Q = kFoldThreads / 2D,
// all of its loads issued at once), then the Q partials of each value are
// added in a fixed order.
constexpr int kFoldThreads = 1024;
template <int D>
__global__ __launch_bounds__(kFoldThreads) void wgrad_fold_kernel(float* slots, float* dwq, float* dwk) {
  constexpr int n = 2 * D;
  constexpr int Q = kFoldThreads / n;  // 4 for D = 128, 8 for D = 64
  constexpr int PER = kWgradSlots / Q;
  static_assert(kWgradSlots % Q == 0, "every thread of the fold sums the same number of slots");
  __shared__ float part[kFoldThreads];
  const int i = threadIdx.x % n, q = threadIdx.x / n;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = slots[(q + j * Q) * n + i];
#pragma unroll
  for (int j = 0; j < PER; ++j) slots[(q + j * Q) * n + i] = 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < PER; ++j) s += v[j];
  part[threadIdx.x] = s;
  __syncthreads();
  if (q == 0) {
#pragma unroll
    for (int r = 1; r < Q; ++r) s += part[r * n + i];
    if (i < D) dwq[i] = s;
    else dwk[i - D] = s;
  }
}

// Weight grads of an empty batch: zero (the workspace is left as it was, zero).
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
  int64_t T;
  const int32_t* bt;
  int32_t bt_stride;
  int32_t tokens_per_req;
  int32_t page_size;
  int32_t num_pages;
  double turns[kMaxPairs];  // turns per position of the 32 rotated pairs
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
  const double tpp = a.turns[lane % (ROPE_D / 2)];

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

// ------------------------------------------------------------------ RoPE in place

// The q path's rotation of each head's rope part ("rope_into" of the MLA
// drafter layer): x [T, heads, head_stride] bf16, the R values at rope_off of
// every head rotated in place at the token's position; nothing else is read
// or written.  One wave per token; LPH = R/8 lanes per head in mirror chunk
// order, HPI = 64/LPH heads per wave iteration.
struct RopeArgs {
  uint8_t* x;
  int64_t T;
  int64_t t0;  // first token of this launch (a large batch takes several launches)
  int64_t token_bytes;
  int32_t head_bytes;
  int32_t rope_off_bytes;
  int32_t heads;
  int32_t iters;  // ceil(heads / HPI)
  const int32_t* pos;
  double turns[kMaxPairs];
};

template <int R>
__global__ __launch_bounds__(kBlockThreads) void rope_inplace_kernel(const RopeArgs a) {
  constexpr int LPH = R / 8, HPI = kWave / LPH;
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & (LPH - 1);
  const int hs = lane / LPH;
  const int c = chunk_of_lane<LPH>(li);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int64_t t = a.t0 + static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (t >= a.T) return;  // wave-uniform
  const double tpp = a.turns[lane % (R / 2)];
  const int32_t p = a.pos[t];
  float cs[8], sn[8];
  unit_cos_sin<8, LPH>(p, tpp, c, cs, sn);
  uint8_t* base = a.x + t * a.token_bytes + a.rope_off_bytes + c * 16;
  for (int it = 0; it < a.iters; ++it) {
    const int h = it * HPI + hs;
    if (h < a.heads) {  // the partner lane belongs to the same head, so it takes the same branch
      uint8_t* ptr = base + static_cast<int64_t>(h) * a.head_bytes;
      float k[8], z[8];
      unpack(ld16(ptr), k);
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = fmaf(k[e], cs[e], partner<LPH>(k[e]) * sn[e]);
      st16(ptr, pack(z));
    }
  }
}

}  // namespace qkvnr
