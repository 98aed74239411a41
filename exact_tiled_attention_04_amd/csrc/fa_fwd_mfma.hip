// Exact attention forward, bf16/fp16 inputs, on CDNA4 matrix cores (gfx950).
//
// What is computed is standard attention with a scale and a mask (the
// "AS-IS" diagram of the Flash Attention page, heepie.pages.dev): per query
// row, softmax over the visible keys of scale * q.k, then the
// probability-weighted sum of V rows.  How it is computed follows that page's
// "TO-BE" diagram and tiling section, and the FlashAttention-2 (PL) article's
// three changes ("Architektura techniczna i zasady działania"):
//
//   * one workgroup per (batch, query head, block of 128 query rows), so one
//     head's work spreads over many compute units (section 2 of the article);
//   * inside the workgroup each of the 4 wavefronts owns 32 query rows
//     outright, so the softmax row statistics never travel through LDS
//     (section 3);
//   * K and V stream through LDS in tiles of 64 keys; the 128 x 64 score tile
//     lives only in registers and never reaches device memory;
//   * an online softmax (FlashAttention quiz, question 4) keeps a running
//     row max m and row sum l; when m grows the partial output is rescaled;
//   * non-matmul work is kept small (section 1): the scale and log2(e) are
//     folded into one multiply-add feeding exp2, the final 1/l is a single
//     multiply per output element, and the rescale of the partial output is
//     skipped when no row max in the wavefront moved.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_{bf16,f16}: A 32x16, B 16x32,
// C 32x32 fp32; lane l holds A[l%32][8*(l/32)+j], B[8*(l/32)+j][l%32] for
// j < 8, and C[8*(i/4)+4*(l/32)+i%4][l%32] for i < 16):
//
//   S^T (keys x queries) = K Q^T   A = K rows straight from LDS (16-byte
//                                  reads), B = this lane's query row, kept in
//                                  registers for the whole key loop.
//   O^T (dims x queries) += V^T P^T
//                                  B = P^T is the S^T accumulator itself after
//                                  exp2 and rounding: the lane already holds 8
//                                  keys of its own query.  A = V^T comes from
//                                  row-major V in LDS through the gfx950
//                                  transposing LDS read (ds_read_b64_tr_b16),
//                                  with the key order permuted to match which
//                                  8 keys each half-wave holds.
//
// With queries along the accumulator columns, every lane owns one query: the
// row max and row sum need one exchange between the two half-waves
// (v_permlane32_swap) and the rescale and 1/l are per-lane scalars.
#include "fa_internal.h"
#include "fa_mfma_common.h"

#include <climits>
#include <type_traits>

namespace fa {
namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kThreads = kWaveSize * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBR = kWaves * kRowsPerWave;  // query rows per workgroup
#ifndef FA_KEYS_PER_TILE
#define FA_KEYS_PER_TILE 64
#endif
#ifndef FA_V_BUFFERS
#define FA_V_BUFFERS 2
#endif
#ifndef FA_WAVES_PER_SIMD
#define FA_WAVES_PER_SIMD 2
#endif
constexpr int kBC = FA_KEYS_PER_TILE;       // keys per K/V tile (32 or 64)
constexpr int kHalves = kBC / 32;           // 32-key score blocks per tile
constexpr int kKBufs = 3;                   // LDS buffers for K (K travels two tiles ahead)
constexpr int kVBufs = FA_V_BUFFERS;        // 2: V one tile ahead; 3: two tiles ahead
constexpr int kWavesPerSimd = FA_WAVES_PER_SIMD;
static_assert(kBC == 32 || kBC == 64, "tile width");
static_assert(kVBufs == 2 || kVBufs == 3, "V buffering");
constexpr float kLn2 = 0.69314718055994531f;

template <int D>
struct Shape {
  static constexpr int kChunks = D / 8;     // 16-byte chunks per row
  static constexpr int kSteps = D / 16;     // MFMA k-steps over the head dimension
  static constexpr int kOutTiles = D / 32;  // 32-wide output channel tiles
  static constexpr int kRowBytes = 2 * D;
  // one wave-wide 16-byte-per-lane load moves 1 KiB = this many rows
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;
  static constexpr int kLoadsPerWave = kBC / kRowsPerLoad / kWaves;
  static_assert(kBC % (kRowsPerLoad * kWaves) == 0, "tile must split evenly over the wavefronts");
};

// LDS layouts.  Both tiles are row-major [key][dim]; the 16-byte chunks of a
// row are permuted by an XOR with a function of the row, chosen (by bank-
// conflict counts on gfx950, whose LDS serves 256 bytes per clock) so that the
// reads of the hot loop are conflict-free:
//   K, read 16 bytes per lane with the 32 lanes of a half-wave on 32
//     consecutive rows: D=128 chunk ^ (row mod 16); D=64 (two rows per 256
//     bytes) chunk ^ ((row / 2) mod 8).
//   V, read through the transposing load with each 16-lane group on 4
//     consecutive rows x 32 bytes: D=128 chunk ^ 4*(row mod 4); D=64
//     chunk ^ 2*(row mod 4).
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? ((row & 3) << 2) : ((row & 3) << 1);
}
template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * D + ((chunk ^ k_swz<D>(row)) << 3);
}
template <int D>
__device__ __forceinline__ int v_off(int row, int col) {
  return row * D + (((col >> 3) ^ v_swz<D>(row)) << 3) + (col & 7);
}

// Per-lane byte offsets (within one tile) of this lane's pieces of the
// direct-to-LDS copies.  Each wave moves kLoadsPerWave 1-KiB pieces of each
// tensor per tile: lane l fills LDS bytes 16l..16l+15 of its piece, so it
// fetches the logical chunk that the swizzle maps there.
template <int D>
struct LoadOffsets {
  int k[Shape<D>::kLoadsPerWave];
  int v[Shape<D>::kLoadsPerWave];
  // row_bytes: distance between consecutive keys of one head in device
  // memory (2d for [B][H][N][d]; 2 * Hkv * d for packed [tokens][Hkv][d])
  __device__ __forceinline__ void init(int wave, int lane, int row_bytes) {
    using S = Shape<D>;
#pragma unroll
    for (int u = 0; u < S::kLoadsPerWave; ++u) {
      const int piece = wave * S::kLoadsPerWave + u;
      const int row = piece * S::kRowsPerLoad + lane / S::kChunks;
      const int pch = lane % S::kChunks;  // physical chunk this lane fills
      k[u] = row * row_bytes + ((pch ^ k_swz<D>(row)) << 4);
      v[u] = row * row_bytes + ((pch ^ v_swz<D>(row)) << 4);
    }
  }
};

// Start copying key tile t of K (or V) from device memory straight into LDS
// (buffer loads with the LDS destination; no registers).  The tile's start
// is a wave-uniform byte offset.  Rows past the end of the sequence lie
// outside the buffer's range and arrive as zeros.
template <int D>
__device__ __forceinline__ void copy_tile_async(__amdgpu_buffer_rsrc_t r, const int* lane_off,
                                                unsigned short* dst, int t, int wave, int row_bytes) {
  using S = Shape<D>;
  const int tile_bytes = t * (kBC * row_bytes);
#pragma unroll
  for (int u = 0; u < S::kLoadsPerWave; ++u) {
    const int piece = wave * S::kLoadsPerWave + u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + piece * 512), 16, lane_off[u],
                                             tile_bytes, 0, 0);
  }
}


// PV MFMAs by which the transposing V reads run ahead of their MFMA.
constexpr int kPvReadLead = 4;

// A row's running max may lag the true max by up to this much (log2 units)
// before the partial output is rescaled; probabilities then stay <= 2^8.
constexpr float kRescaleSlack = 8.0f;

// Per-lane constants of one workgroup's key loop.
template <int D>
struct LoopCtx {
  __amdgpu_buffer_rsrc_t rk, rv;  // this (batch, kv head)'s K and V, bounded to N rows
  LoadOffsets<D> off;
  int N, wl, t_beg, t_end;
  int wave, lane, l32, hh;
  int wq0, wq1;                   // first and last valid row of the wavefront
  int shift;                      // key position of query row 0 (0 unless fewer queries than keys)
  int kv_row_bytes;               // distance between consecutive keys of one head
  int vis_lo;                     // first visible key of this lane's row
  unsigned vis_span;              // visible keys: vis_lo .. vis_lo + vis_span
  int v_row_lane, v_col_lane;     // lane geometry of the transposing V read
  bool causal;
  float c;                        // scale * log2(e)
};

// Running state of the lane's query row.
template <int D>
struct RowState {
  u32x4 qf[Shape<D>::kSteps];         // q row as the B operand
  f32x16 oacc[Shape<D>::kOutTiles];   // unnormalised O^T columns
  float m_use;                        // max used in the exponents (scale*log2(e) units)
  float l_run;                        // running sum of exp2(. - m_use), this half-wave's keys
};

// Scores of key tile t: S^T = K Q^T; s[h] holds keys kBC*t + 32h .. +31.
template <typename E, int D>
__device__ __forceinline__ void tile_scores(const unsigned short* __restrict__ cK, const LoopCtx<D>& x,
                                            const RowState<D>& st, f32x16 (&s)[kHalves]) {
#pragma unroll
  for (int h = 0; h < kHalves; ++h) s[h] = f32x16{};
#pragma unroll
  for (int kc = 0; kc < Shape<D>::kSteps; ++kc) {
#pragma unroll
    for (int h = 0; h < kHalves; ++h) {
      const u32x4 a = *(const u32x4*)(cK + k_off<D>(32 * h + x.l32, 2 * kc + x.hh));
      s[h] = E::mma(a, st.qf[kc], s[h]);
    }
  }
}

// Mask tile t when it crosses the causal diagonal, the window edge or the
// sequence end for some row of the wavefront: key kb + off is visible iff
// 0 <= kb + off - vis_lo <= vis_span.
template <int D>
__device__ __forceinline__ void tile_mask(const LoopCtx<D>& x, int t, f32x16 (&s)[kHalves]) {
  const int kb = t * kBC;
  const int ke = kb + kBC - 1;
  const bool need_mask = (ke >= x.N) || (x.causal && ke > x.wq0 + x.shift) ||
                         (x.wl >= 0 && kb < x.wq1 + x.shift - x.wl);
  if (!need_mask) return;
  const int base = kb - x.vis_lo + 4 * x.hh;
#pragma unroll
  for (int h = 0; h < kHalves; ++h) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int off = 32 * h + 8 * (i >> 2) + (i & 3);
      s[h][i] = ((unsigned)(base + off) <= x.vis_span) ? s[h][i] : -INFINITY;
    }
  }
}

// Maximum of N values as a tree of three-input maxima (v_max3_f32): every
// level folds groups of three and carries up to two leftovers, so 32 values
// take 16 instructions instead of 31 two-input ones.
template <int N>
__device__ __forceinline__ float max_tree(const float (&a)[N]) {
  if constexpr (N == 1) {
    return a[0];
  } else if constexpr (N == 2) {
    return __builtin_fmaxf(a[0], a[1]);
  } else {
    constexpr int G = N / 3, M = G + N % 3;
    float b[M];
#pragma unroll
    for (int i = 0; i < G; ++i) b[i] = __builtin_fmaxf(__builtin_fmaxf(a[3 * i], a[3 * i + 1]), a[3 * i + 2]);
#pragma unroll
    for (int i = 0; i < N % 3; ++i) b[G + i] = a[3 * G + i];
    return max_tree<M>(b);
  }
}

// Online softmax of one score tile (base 2, scale folded into the
// exponent): turns s0/s1 into the P^T operands pf, updates the row's
// reference max and sum, and returns the factor the partial output must be
// multiplied by (1 unless the reference max moved).
template <typename E, int D>
__device__ __forceinline__ float tile_softmax(const LoopCtx<D>& x, RowState<D>& st, f32x16 (&s)[kHalves],
                                              u32x4* pf) {
  // row max over the lane's 16*kHalves scores
  float sv[16 * kHalves];
#pragma unroll
  for (int h = 0; h < kHalves; ++h) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[16 * h + i] = s[h][i];
  }
  float mx = max_tree(sv);
  float mlo, mhi;
  half_pair(mx, mlo, mhi);
  mx = fmaxf(mlo, mhi) * x.c;
  // Move the reference max only when the true max got ahead of it by more
  // than the slack (always on the first visible key).  No NaN can arise:
  // when bumped, mx is finite and m_use - mx is finite or -inf; otherwise
  // the factor is exactly 1.
  const bool bump = mx > st.m_use + kRescaleSlack;
  const float alpha = bump ? __builtin_amdgcn_exp2f(st.m_use - mx) : 1.f;
  st.m_use = bump ? mx : st.m_use;
  const float m_exp = (st.m_use == -INFINITY) ? 0.f : st.m_use;  // nothing visible yet
  float rs = 0.f;
#pragma unroll
  for (int h = 0; h < kHalves; ++h) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[h][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][i], x.c, -m_exp));
      rs += s[h][i];
    }
  }
  st.l_run = __builtin_fmaf(st.l_run, alpha, rs);
  // P^T operands: the lane's own probabilities, 8 keys per k-step
#pragma unroll
  for (int h = 0; h < kHalves; ++h) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      pf[2 * h + j] = u32x4{E::pack2(s[h][8 * j + 0], s[h][8 * j + 1]), E::pack2(s[h][8 * j + 2], s[h][8 * j + 3]),
                            E::pack2(s[h][8 * j + 4], s[h][8 * j + 5]), E::pack2(s[h][8 * j + 6], s[h][8 * j + 7])};
  }
  return alpha;
}

// O^T += V^T P^T for one tile.  k-step mc covers keys 16mc..16mc+15 in the
// order the score accumulator hands them over: half-wave hh holds keys
// 16mc + 4hh + {0..3} and 16mc + 8 + 4hh + {0..3}.  The k-steps are the outer
// loop, so consecutive products share their P^T operand (measured ~0.7%
// faster than output tile by output tile, bit-identical).
template <typename E, int D>
__device__ __forceinline__ void tile_pv(const unsigned short* __restrict__ vC, const LoopCtx<D>& x,
                                        RowState<D>& st, const u32x4* pf) {
#pragma unroll
  for (int mc = 0; mc < 2 * kHalves; ++mc) {
#pragma unroll
    for (int ct = 0; ct < Shape<D>::kOutTiles; ++ct) {
      const int col = 32 * ct + x.v_col_lane;
      const int ra = 16 * mc + x.v_row_lane;
      const s16x4 lo = lds_read_tr(vC, v_off<D>(ra, col));
      const s16x4 hi = lds_read_tr(vC, v_off<D>(ra + 8, col));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 a = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
      st.oacc[ct] = E::mma(a, pf[mc], st.oacc[ct]);
    }
  }
}

__device__ __forceinline__ void rescale_if_needed(float alpha, f32x16* oacc, int tiles) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
    for (int ct = 0; ct < tiles; ++ct) oacc[ct] *= alpha;
  }
}

// One step of the key loop, software-pipelined so that the vector units'
// softmax of tile t runs while the matrix cores accumulate P(t-1) V(t-1):
//   1. S(t) = K(t) Q^T on the matrix cores, at raised wave priority: while
//      this wave issues its score MFMAs, the other wave on the SIMD (from the
//      other workgroup) fills the vector units with its softmax;
//   2. softmax(S(t)) -> P(t), interleaved with O += P(t-1) V(t-1), after O is
//      brought to the reference max that P(t-1) was computed with.
// K(t) and V(t-1) are in LDS when the step starts.  The step first starts
// copying V into vN (V(t) with two V buffers, V(t+1) with three; the buffer
// held V(t-2)), then K(t+2) into kN (K(t-1)'s buffer); both buffers were
// last read in step t-1.  K thus travels two steps ahead, V one or two.  The buffer pointers are restrict-qualified: copy targets are never
// read in this step, which lets the LDS reads proceed while copies are in
// flight.
template <typename E, int D, bool kHasPrev>
__device__ __forceinline__ void pipeline_step(const unsigned short* __restrict__ kC,  // holds K(t)
                                              unsigned short* __restrict__ kN,        // gets K(t+2)
                                              const unsigned short* __restrict__ vC,  // holds V(t-1)
                                              unsigned short* __restrict__ vN,        // gets V(t)
                                              const LoopCtx<D>& x, RowState<D>& st, u32x4* pf_prev,
                                              float& alpha_prev, int t) {
  using S = Shape<D>;
  // V(t) (two V buffers) or V(t+1) (three); past the end: zeros, never read
  copy_tile_async<D>(x.rv, x.off.v, vN, t + kVBufs - 2, x.wave, x.kv_row_bytes);
  copy_tile_async<D>(x.rk, x.off.k, kN, t + 2, x.wave, x.kv_row_bytes);

  f32x16 s[kHalves];
  __builtin_amdgcn_s_setprio(2);
  tile_scores<E, D>(kC, x, st, s);
  __builtin_amdgcn_s_setprio(0);
  tile_mask<D>(x, t, s);

  // P(t-1) was computed with the reference max as it stood after tile t-1;
  // O still carries the scale before it: bring O to that scale first.
  if (kHasPrev) rescale_if_needed(alpha_prev, st.oacc, S::kOutTiles);

  u32x4 pf[2 * kHalves];
  const float alpha = tile_softmax<E, D>(x, st, s, pf);
  if (kHasPrev) {
    tile_pv<E, D>(vC, x, st, pf_prev);
    // interleave: each PV MFMA follows a slice of the softmax work, and its
    // two transposing reads were issued kPvReadLead MFMAs earlier
    constexpr int kPv = 2 * kHalves * S::kOutTiles;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvReadLead, 0);  // LDS read
#pragma unroll
    for (int g = 0; g < kPv; ++g) {
      if (g + kPvReadLead < kPv) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);                    // VALU
    }
  }
#pragma unroll
  for (int j = 0; j < 2 * kHalves; ++j) pf_prev[j] = pf[j];
  alpha_prev = alpha;
}

// Wait until at most this wave's newest kInFlight copies are outstanding,
// then for every wave to do so: the copies the next step reads have landed
// and every wave is done with the buffers the next copies will overwrite.
// (A plain workgroup barrier would also wait for every outstanding copy; the
// memory clobber keeps the compiler from moving memory operations across.)
template <int kInFlight>
__device__ __forceinline__ void tile_barrier() {
  static_assert(kInFlight >= 0 && kInFlight < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kInFlight) : "memory");
}

// kVarlen: sequences of different lengths packed as q [total_q][Hq][d],
// k, v [total_k][Hkv][d], sequence b owning rows cu_q[b] .. cu_q[b+1]-1 (and
// keys cu_k[b] .. cu_k[b+1]-1); its Lq query rows stand at the end of its Lk
// keys (row i at position Lk - Lq + i), lse is [Hq][total_q], and rows that
// see no key get o = 0 and lse = -inf.  Otherwise one N for queries and keys
// in [B][H][N][d].
template <typename E, int D, bool kVarlen>
__global__ void __launch_bounds__(kThreads, kWavesPerSimd) fwd_mfma_kernel(FwdParams p) {
  using S = Shape<D>;
  // three K and two V buffers, as separate objects (80 KiB at d = 128, so two
  // workgroups share a compute unit)
  __shared__ __attribute__((aligned(16))) unsigned short sK0[kBC * D];
  __shared__ __attribute__((aligned(16))) unsigned short sK1[kBC * D];
  __shared__ __attribute__((aligned(16))) unsigned short sK2[kBC * D];
  __shared__ __attribute__((aligned(16))) unsigned short sV0[kBC * D];
  __shared__ __attribute__((aligned(16))) unsigned short sV1[kBC * D];
#if FA_V_BUFFERS == 3
  __shared__ __attribute__((aligned(16))) unsigned short sV2[kBC * D];
#else
  unsigned short* const sV2 = sV0;  // never used with two V buffers
#endif

  LoopCtx<D> x;
  const int tid = threadIdx.x;
  x.lane = tid & (kWaveSize - 1);
  x.wave = __builtin_amdgcn_readfirstlane(tid / kWaveSize);  // wave-uniform: keep it scalar
  x.l32 = x.lane & 31;
  x.hh = x.lane >> 5;

  WorkItem it;
  if constexpr (kVarlen) {
    // Packed sequences of different lengths cost very different amounts, so
    // instead of contiguous slices of the (sequence, key/value head) groups,
    // XCD x (workgroup id mod 8) takes groups x, x + 8, x + 16, ...: every
    // XCD gets a spread of lengths.  A group's query blocks (and the query
    // heads sharing its key/value head) stay on one XCD, heaviest block
    // first, so its K/V tiles are shared through that XCD's L2.  The grid
    // holds 8 * ceil(groups / 8) groups; the missing ones return at once.
    const int xcd = blockIdx.x % 8;
    const int r = blockIdx.x / 8;
    const int per_group = p.group * p.n_qblocks;
    const int j = r / per_group;
    const int w = r - j * per_group;
    const int gidx = 8 * j + xcd;
    if (gidx >= p.B * p.Hkv) return;
    const int qrank = w / p.group;
    const int hg = w - qrank * p.group;
    const int gb = gidx / p.Hkv;
    it.bh = gb * p.Hq + (gidx - gb * p.Hkv) * p.group + hg;
    it.qb = p.causal ? (p.n_qblocks - 1 - qrank) : qrank;
  } else {
    it = decode_work_item(p, blockIdx.x);
  }
  const int b = it.bh / p.Hq;
  const int hq = it.bh - b * p.Hq;
  const int hk = hq / p.group;
  int Nq, N;                // query rows and keys of this sequence
  long long q_head, kv_head;  // element offsets of this head's row 0
  int q_stride;             // elements between consecutive query rows
  int q_row0 = 0;           // packed: the sequence's first row in q
  if constexpr (kVarlen) {
    // offsets clamped to the packed tensors, lengths to the launch's maxima,
    // so inconsistent offsets can never address outside the buffers
    typedef __attribute__((address_space(4))) const int cint;
    const int qa = min(max(((cint*)p.cu_q)[b], 0), p.total_q);
    const int qz = min(max(((cint*)p.cu_q)[b + 1], qa), p.total_q);
    const int ka = min(max(((cint*)p.cu_k)[b], 0), p.total_k);
    const int kz = min(max(((cint*)p.cu_k)[b + 1], ka), p.total_k);
    Nq = min(qz - qa, p.N);
    N = min(kz - ka, p.max_k);
    if (it.qb * kBR >= Nq) return;  // the whole workgroup: past this sequence's rows
    x.shift = N - Nq;
    q_row0 = qa;
    q_head = ((long long)qa * p.Hq + hq) * D;
    kv_head = ((long long)ka * p.Hkv + hk) * D;
    q_stride = p.Hq * D;
    x.kv_row_bytes = 2 * p.Hkv * D;
  } else {
    Nq = N = p.N;
    x.shift = 0;
    q_head = (long long)it.bh * N * D;
    kv_head = ((long long)b * p.Hkv + hk) * N * D;
    q_stride = D;
    x.kv_row_bytes = S::kRowBytes;
  }
  x.off.init(x.wave, x.lane, x.kv_row_bytes);
  x.N = N;
  const unsigned short* __restrict__ qg = (const unsigned short*)p.q + q_head;
  const int head_bytes = kVarlen ? (N > 0 ? (N - 1) * x.kv_row_bytes + S::kRowBytes : 0) : N * S::kRowBytes;
  x.rk = __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned short*)p.k + kv_head), 0, head_bytes,
                                           kBufferFlags);
  x.rv = __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned short*)p.v + kv_head), 0, head_bytes,
                                           kBufferFlags);

  x.causal = p.causal != 0;
  x.wl = p.window_left;
  x.c = p.scale_log2;
  const int q0 = it.qb * kBR;
  x.wq0 = q0 + x.wave * kRowsPerWave;
  x.wq1 = min(Nq, x.wq0 + kRowsPerWave) - 1;
  const int myq = x.wq0 + x.l32;  // this lane's query row

  // Key tiles this workgroup needs: causal stops at its last row, a window
  // starts window_left keys before its first row.
  const int kend = x.causal ? min(N, q0 + kBR + x.shift) : N;
  const int kbeg = x.wl >= 0 ? max(0, q0 + x.shift - x.wl) : 0;
  x.t_beg = kbeg / kBC;
  x.t_end = (kend + kBC - 1) / kBC;

  // Visible keys of this lane's row form one range [vis_lo, vis_lo + vis_span].
  const int pos = myq + x.shift;
  x.vis_lo = x.wl >= 0 ? max(0, pos - x.wl) : 0;
  const int vis_hi = x.causal ? min(pos, N - 1) : N - 1;
  x.vis_span = (unsigned)(vis_hi - x.vis_lo);
  if constexpr (kVarlen) {
    if (vis_hi < x.vis_lo) {  // a row that sees no key: nothing is visible
      x.vis_lo = INT_MAX / 2;
      x.vis_span = 0;
    }
    if (kend <= kbeg) {  // no row of the workgroup sees a key
      if (myq < Nq) {
        unsigned short* og = (unsigned short*)p.o + q_head + (long long)myq * q_stride;
#pragma unroll
        for (int c = 0; c < D / 4; c += 2) *(u32x2*)(og + 4 * (c + x.hh)) = u32x2{0u, 0u};
        if (x.hh == 0 && p.lse != nullptr) p.lse[(long long)hq * p.total_q + q_row0 + myq] = -INFINITY;
      }
      return;
    }
  }

  const int g16 = x.lane >> 4;
  const int gi = x.lane & 15;
  x.v_row_lane = 4 * x.hh + (gi >> 2);
  x.v_col_lane = 16 * (g16 & 1) + 4 * (gi & 3);

  RowState<D> st;
#pragma unroll
  for (int kc = 0; kc < S::kSteps; ++kc) {
    if (myq < Nq)
      st.qf[kc] = q_signed16(*(const u32x4*)(qg + (long long)myq * q_stride + 16 * kc + 8 * x.hh), p.q_sign);
    else
      st.qf[kc] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int ct = 0; ct < S::kOutTiles; ++ct) st.oacc[ct] = f32x16{};
  st.m_use = -INFINITY;
  st.l_run = 0.f;

  // With i = t - t_beg: K(t) lives in K buffer i % 3, V(t) in V buffer
  // i % kVBufs.
  // The step loop is unrolled six ways so every buffer choice is a
  // compile-time constant (LDS addresses fold into instruction offsets).
  auto kbuf = [&](int j) { return j == 0 ? sK0 : (j == 1 ? sK1 : sK2); };
  auto vbuf = [&](int j) { return j == 0 ? sV0 : (j == 1 ? sV1 : sV2); };
  // copies a wave may leave in flight at a step's barrier: with two V
  // buffers the previous step's K copy (its last), with three all of the
  // previous step's copies
  constexpr int kInFlight = (kVBufs - 1) * S::kLoadsPerWave;
  const int t0 = x.t_beg;
  copy_tile_async<D>(x.rk, x.off.k, sK0, t0, x.wave, x.kv_row_bytes);
  copy_tile_async<D>(x.rk, x.off.k, sK1, t0 + 1, x.wave, x.kv_row_bytes);  // past the end: zeros, never read
  if (kVBufs == 3) copy_tile_async<D>(x.rv, x.off.v, sV0, t0, x.wave, x.kv_row_bytes);
  u32x4 pf_prev[2 * kHalves];
  float alpha_prev = 1.f;
  tile_barrier<0>();
  pipeline_step<E, D, false>(sK0, sK2, vbuf(kVBufs - 1), vbuf(kVBufs == 3 ? 1 : 0), x, st, pf_prev, alpha_prev,
                             t0);
  auto step = [&](auto uc, int t) {
    constexpr int u = decltype(uc)::value;  // (t - t0) % 6
    // reads K(t) and V(t-1); fills the buffers of K(t-1) and V(t-2)
    constexpr int vc = (u + kVBufs - 1) % kVBufs;
    constexpr int vn = kVBufs == 3 ? (u + 1) % 3 : u % 2;
    tile_barrier<kInFlight>();
    pipeline_step<E, D, true>(kbuf(u % 3), kbuf((u + 2) % 3), vbuf(vc), vbuf(vn), x, st, pf_prev, alpha_prev,
                              t);
  };
  for (int t = t0 + 1; t < x.t_end; t += 6) {
    step(std::integral_constant<int, 1>{}, t);
    if (t + 1 < x.t_end) step(std::integral_constant<int, 2>{}, t + 1);
    if (t + 2 < x.t_end) step(std::integral_constant<int, 3>{}, t + 2);
    if (t + 3 < x.t_end) step(std::integral_constant<int, 4>{}, t + 3);
    if (t + 4 < x.t_end) step(std::integral_constant<int, 5>{}, t + 4);
    if (t + 5 < x.t_end) step(std::integral_constant<int, 0>{}, t + 5);
  }
  // drain: P(t_end-1) V(t_end-1); wait for every copy, so that none is still
  // in flight into LDS when the workgroup ends
  tile_barrier<0>();
  rescale_if_needed(alpha_prev, st.oacc, S::kOutTiles);
  const int rl = (x.t_end - 1 - t0) % kVBufs;
  if (rl == 0)
    tile_pv<E, D>(sV0, x, st, pf_prev);
  else if (rl == 1)
    tile_pv<E, D>(sV1, x, st, pf_prev);
  else
    tile_pv<E, D>(sV2, x, st, pf_prev);

  // ---- epilogue: one division per row, store O and the logsumexp
  float llo, lhi;
  half_pair(st.l_run, llo, lhi);
  const float l_tot = llo + lhi;
  if (myq < Nq) {
    const bool seen = !kVarlen || l_tot > 0.f;  // only packed rows can see no key
    const float inv = seen ? 1.f / l_tot : 0.f;
    unsigned short* og = (unsigned short*)p.o + q_head + (long long)myq * q_stride;
#pragma unroll
    for (int ct = 0; ct < S::kOutTiles; ++ct) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const u32x2 w = u32x2{E::pack2(st.oacc[ct][4 * gq + 0] * inv, st.oacc[ct][4 * gq + 1] * inv),
                              E::pack2(st.oacc[ct][4 * gq + 2] * inv, st.oacc[ct][4 * gq + 3] * inv)};
        *(u32x2*)(og + 32 * ct + 8 * gq + 4 * x.hh) = w;
      }
    }
    if (x.hh == 0 && p.lse != nullptr) {
      const float lse = seen ? (st.m_use + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
      if constexpr (kVarlen)
        p.lse[(long long)hq * p.total_q + q_row0 + myq] = lse;
      else
        p.lse[(long long)it.bh * N + myq] = lse;
    }
  }
}

template <typename E, int D>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const FwdParams p = make_params(a, kBR);
  if (p.cu_q) {
    // eight XCDs times the rounds of (sequence, key/value head) groups
    const long long groups = (long long)p.B * p.Hkv;
    const long long grid = 8 * ((groups + 7) / 8) * p.group * p.n_qblocks;
    hipLaunchKernelGGL((fwd_mfma_kernel<E, D, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((fwd_mfma_kernel<E, D, false>), dim3(p.total_items), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch<Bf16, 64>(a, stream) : launch<Bf16, 128>(a, stream);
}

hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch<F16, 64>(a, stream) : launch<F16, 128>(a, stream);
}

long long mfma_rows_per_workgroup() { return kBR; }

}  // namespace fa
