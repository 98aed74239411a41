// Exact attention backward (dQ, dK, dV), bf16/fp16 inputs, on CDNA4 matrix
// cores (gfx950).
//
// Given the forward's inputs, its output O and row logsumexp, and an upstream
// gradient dO, the gradients of standard attention are (per batch and query
// head, key/value head g(h)):
//
//   P    = exp(scale * Q K^T - lse)     recomputed, never stored
//   dV  += P^T dO                       (summed over the query heads of g)
//   dP   = dO V^T
//   dS   = P * (dP - D),   D_i = sum_c dO_ic O_ic
//   dQ   = scale * dS K
//   dK  += scale * dS^T Q               (summed over the query heads of g)
//
// The probabilities are rebuilt from Q, K and the saved row statistics rather
// than kept from the forward: the recomputation that the Flash Attention page
// (heepie.pages.dev, tiling section) credits with trading a few extra FLOPs for
// far less HBM traffic.  D_i uses the forward's output: for exact O it equals
// sum_j P_ij dP_ij, the row term of the softmax Jacobian.
//
// Three launches, no atomics, bit-reproducible:
//   1. prep: -D_i and lse_i * log2(e) for every row, into the caller's
//      workspace (-D starts the dP accumulators, which then come out of the
//      matrix cores as dP - D);
//   2. dK/dV: one workgroup per (batch, key/value head, block of 128 keys,
//      64 at d = 64); each pair of its wavefronts owns 32 keys, takes their
//      K and V rows as MFMA operands (from registers at d = 64, from LDS at
//      d = 128) and keeps their dK^T, dV^T in accumulators, while 64-row
//      tiles of Q, dO, lse, D of every query head in the group stream
//      through LDS;
//   3. dQ: one workgroup per (batch, query head, block of 128 queries), the
//      forward's layout: each wavefront owns 32 queries, 64-key tiles of K and
//      V stream through LDS.
//
// Packed sequences of different lengths (kPacked) run the same kernels with
// per-sequence offsets and lengths, token-major rows ([token][head][d], so
// row strides of H * d elements) and each sequence's queries standing at the
// end of its keys (query i at key position i + Lk - Lq); the row terms and
// lse are [Hq][total_q].  A row that sees no key has lse = -inf and gets
// P = 0 everywhere.
//
// Matrix-core mapping as in the forward (v_mfma_f32_32x32x16; lane l holds
// A[l%32][8*(l/32)+j], B[8*(l/32)+j][l%32], C[8*(i/4)+4*(l/32)+i%4][l%32]):
// every product keeps the wavefront's own rows on the accumulator columns, so
// a score accumulator is directly the B operand of the next product after
// exp2 and rounding, and the streamed tile enters that product through the
// transposing LDS read with the k order permuted to match the accumulator.
// Streamed tiles are read both as 16-byte rows (A operand of a score-like
// product) and through the transposing read, so their LDS swizzle is chosen
// to be conflict-free for both patterns.
#include "fa_internal.h"
#include "fa_mfma_common.h"

namespace fa {
namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kThreads = kWaveSize * kWaves;
constexpr int kRows = 32;                // rows a wavefront owns (queries in dQ, keys in dK/dV)
constexpr int kBlock = kWaves * kRows;   // rows a workgroup owns
constexpr int kTile = 64;                // streamed rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

template <int D, int W = kWaves>
struct Shape {
  static constexpr int kChunks = D / 8;     // 16-byte chunks per row
  static constexpr int kSteps = D / 16;     // MFMA k-steps over the head dimension
  static constexpr int kOutTiles = D / 32;  // 32-wide output tiles over the head dimension
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows per 1-KiB wave-wide load
  static constexpr int kLoadsPerWave = kTile / kRowsPerLoad / W;  // copy share of each of W wavefronts
  static_assert(kTile % (kRowsPerLoad * W) == 0, "tile must split evenly over the wavefronts");
};

// Chunk swizzle of a streamed tile.  Row reads: 16 lanes on 16 consecutive
// rows, one logical chunk; transposing reads: 32 lanes on 4 consecutive rows
// (starting at a multiple of 4) x 4 consecutive chunks.  Both hit 64 distinct
// banks (checked with a bank model): D = 128 (256-byte rows) permutes the
// chunk by the two low row bits into the high chunk bits and the next two row
// bits into the low ones; D = 64 (128-byte rows) does the same with row bit 1
// and row bits 2-3.
template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int row_off(int row, int chunk) {  // element offset of a 16-byte chunk
  return row * D + ((chunk ^ swz<D>(row)) << 3);
}
template <int D>
__device__ __forceinline__ int tr_off(int row, int col) {  // element offset of a 4-element piece
  return row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
}

// Per-lane source offsets of this lane's part of a tile copy: lane l fills
// LDS bytes 16l..16l+15 of its 1-KiB piece, i.e. physical chunk l % kChunks
// of its row, so it fetches the logical chunk the swizzle maps there.  Rows
// lie row_bytes apart in memory (2 D for one head's contiguous rows, more
// for token-major packed sequences).
template <int D, int W = kWaves>
struct CopyOffsets {
  int off[Shape<D, W>::kLoadsPerWave];
  int row_bytes;
  __device__ __forceinline__ void init(int wave, int lane, int rb) {
    using S = Shape<D, W>;
    row_bytes = rb;
#pragma unroll
    for (int u = 0; u < S::kLoadsPerWave; ++u) {
      const int piece = wave * S::kLoadsPerWave + u;
      const int row = piece * S::kRowsPerLoad + lane / S::kChunks;
      const int pch = lane % S::kChunks;
      off[u] = row * rb + ((pch ^ swz<D>(row)) << 4);
    }
  }
};

// Copy rows row0 .. row0+kTile-1 of the tensor behind `r` (bounded to the
// head's rows: rows past the end arrive as zeros) straight into LDS.
template <int D, int W = kWaves>
__device__ __forceinline__ void copy_tile(__amdgpu_buffer_rsrc_t r, const CopyOffsets<D, W>& c,
                                          unsigned short* dst, int row0, int wave) {
  using S = Shape<D, W>;
  // (builtin arguments go through plain ints: the host compilation pass
  // rejects template-dependent expressions in this builtin's operands)
  const int soff = row0 * c.row_bytes;
#pragma unroll
  for (int u = 0; u < S::kLoadsPerWave; ++u) {
    const int piece = wave * S::kLoadsPerWave + u;
    const int voff = c.off[u];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + piece * 512), 16, voff, soff, 0, 0);
  }
}

// Copy kTile floats (rows row0.. of a bounded per-head vector) into LDS:
// one 4-byte load per lane of one wavefront.
__device__ __forceinline__ void copy_vec(__amdgpu_buffer_rsrc_t r, float* dst, int row0, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 4, 4 * lane, 4 * row0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, long long byte_off, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)base + byte_off), 0, bytes, kBufferFlags);
}

// Wait for every copy this wave issued, then for every wave.
__device__ __forceinline__ void barrier_all() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One sequence's rows and, for packed sequences, where they sit: query rows
// qa .. qa+Nq-1 and key rows ka .. ka+Nk-1, query row i at key position
// i + shift (shift = Nk - Nq: the queries are the sequence's last tokens).
// Offsets are clamped to the packed tensors and lengths to the launch's
// maxima, so inconsistent offsets never address outside the buffers.
struct SeqRows {
  int qa, ka, Nq, Nk, shift;
};
template <bool kPacked>
__device__ __forceinline__ SeqRows seq_rows(const BwdParams& p, int b) {
  SeqRows r;
  if constexpr (kPacked) {
    typedef __attribute__((address_space(4))) const int cint;
    r.qa = min(max(((cint*)p.cu_q)[b], 0), p.total_q);
    const int qz = min(max(((cint*)p.cu_q)[b + 1], r.qa), p.total_q);
    r.ka = min(max(((cint*)p.cu_k)[b], 0), p.total_k);
    const int kz = min(max(((cint*)p.cu_k)[b + 1], r.ka), p.total_k);
    r.Nq = min(qz - r.qa, p.N);
    r.Nk = min(kz - r.ka, p.max_k);
  } else {
    r.qa = r.ka = 0;
    r.Nq = r.Nk = p.N;
  }
  r.shift = r.Nk - r.Nq;
  return r;
}

// A = the streamed tile read through the transposing load for k-step mc
// (rows 16mc..16mc+15 in the accumulator's order) and output tile ct.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const unsigned short* __restrict__ t, int mc, int ct, int row_lane,
                                            int col_lane) {
  const int ra = 16 * mc + row_lane;
  const int col = 32 * ct + col_lane;
  const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(t, tr_off<D>(ra, col)));
  const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(t, tr_off<D>(ra + 8, col)));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// 32 x 32 product of 32 streamed rows (32h..32h+31 of the tile, read as
// 16-byte rows) with the wavefront's own rows held as B operands.
template <typename E, int D>
__device__ __forceinline__ f32x16 rows_times_own(const unsigned short* __restrict__ t, int h, int l32, int hh,
                                                 const u32x4* own, f32x16 acc = f32x16{}) {
#pragma unroll
  for (int kc = 0; kc < Shape<D>::kSteps; ++kc) {
    const u32x4 a = *(const u32x4*)(t + row_off<D>(32 * h + l32, 2 * kc + hh));
    acc = E::mma(a, own[kc], acc);
  }
  return acc;
}

// Load a row of 16-bit elements as the wavefront's B operands (lane holds
// elements 16kc + 8hh .. +7 for k-step kc); zero past the end.
template <int D>
__device__ __forceinline__ void load_own_row(const unsigned short* row, bool valid, int hh, u32x4* dst) {
#pragma unroll
  for (int kc = 0; kc < Shape<D>::kSteps; ++kc)
    dst[kc] = valid ? *(const u32x4*)(row + 16 * kc + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
}

// Store an accumulated output row (lane owns the row; element i of tile ct is
// column 32ct + 8(i/4) + 4hh + i%4), multiplied by `mul`.
template <typename E, int D>
__device__ __forceinline__ void store_row(unsigned short* row, const f32x16* acc, float mul, int hh) {
#pragma unroll
  for (int ct = 0; ct < Shape<D>::kOutTiles; ++ct) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const u32x2 w = u32x2{E::pack2(acc[ct][4 * gq + 0] * mul, acc[ct][4 * gq + 1] * mul),
                            E::pack2(acc[ct][4 * gq + 2] * mul, acc[ct][4 * gq + 3] * mul)};
      *(u32x2*)(row + 32 * ct + 8 * gq + 4 * hh) = w;
    }
  }
}

// Pack the 16 fp32 values of one 32-row accumulator into the two B operands
// of the k-steps it covers.
template <typename E>
__device__ __forceinline__ void pack_operands(const float* x, u32x4* dst) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
    dst[j] = u32x4{E::pack2(x[8 * j + 0], x[8 * j + 1]), E::pack2(x[8 * j + 2], x[8 * j + 3]),
                   E::pack2(x[8 * j + 4], x[8 * j + 5]), E::pack2(x[8 * j + 6], x[8 * j + 7])};
}

// ---------------------------------------------------------------------------
// 1. Row terms: -D_i = -sum_c dO_ic O_ic (fp32) and lse_i * log2(e).

template <typename E>
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b);

template <>
__device__ __forceinline__ float dot8<Bf16>(u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    s = __builtin_fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), s);
    s = __builtin_fmaf(__uint_as_float(a[w] & 0xffff0000u), __uint_as_float(b[w] & 0xffff0000u), s);
  }
  return s;
}

template <>
__device__ __forceinline__ float dot8<F16>(u32x4 a, u32x4 b) {
  // (the whole 16 bytes are reinterpreted at once: casting single elements
  // of the dword vector compiled to reads of element 0 only)
  const f16x8 x = __builtin_bit_cast(f16x8, a);
  const f16x8 y = __builtin_bit_cast(f16x8, b);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)x[e], (float)y[e], s);
  return s;
}

template <typename E, int D, bool kPacked>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int c = threadIdx.x % kLanesPerRow;
  float s = 0.f;
  if (row < p.rows) {
    const u32x4 a = *((const u32x4*)((const unsigned short*)p.dout + row * D) + c);
    const u32x4 b = *((const u32x4*)((const unsigned short*)p.o + row * D) + c);
    s = dot8<E>(a, b);
  }
#pragma unroll
  for (int m = kLanesPerRow / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, kLanesPerRow);
  if (row < p.rows && c == 0) {
    // packed: row = token * Hq + head, while lse and the row terms are
    // [Hq][total_q]
    long long idx = row;
    if constexpr (kPacked) {
      const long long t = row / p.Hq;
      idx = (row - t * p.Hq) * p.total_q + t;
    }
    p.delta[idx] = -s;  // stored negated: it initialises the dP accumulators
    // a row that saw no key (lse = -inf) gets P = exp2(s - inf) = 0
    const float l = p.lse[idx];
    p.lse2[idx] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: workgroup = (batch, key/value head, block of keys): 128 keys
// and 8 wavefronts at D = 128, 64 keys and 4 wavefronts at D = 64.
//
// Wavefronts w and w+G (G key groups) own the same 32 keys (group w % G) and
// take opposite 32-query halves of every 64-row query tile, so the two share
// a SIMD and hide each other's latencies without repeating any product.
// Each keeps partial dK^T, dV^T for its keys; the halves are summed through
// LDS once at the end.  At D = 64 (167 registers) the smaller workgroups let
// three of them share a compute unit, so a SIMD interleaves wavefronts of
// three independent workgroups instead of two of one (measured 10.8% faster
// on the whole backward of the d = 64 workload, bit-identical: each key's
// sums see the same tiles in the same order); at D = 128 (238 registers, the
// block's K and V rows in LDS) one 8-wavefront workgroup per compute unit
// is what the registers and LDS allow.

#ifndef FA_BWD_D64_WAVES
#define FA_BWD_D64_WAVES 4
#endif
// wavefronts of a dK/dV workgroup: two per key group of 32 keys
template <int D>
constexpr int kDkvWaves = D == 64 ? FA_BWD_D64_WAVES : 8;
template <int D>
constexpr int kDkvGroups = kDkvWaves<D> / 2;
template <int D>
constexpr int kDkvBlock = kRows * kDkvGroups<D>;  // keys per workgroup
template <int D>
constexpr int kDkvWavesPerSimd = kDkvWaves<D> == 4 ? 3 : 2;

// At D = 128 the K and V rows of the workgroup's keys are read from LDS as
// MFMA operands instead of living in registers (32 VGPRs a lane each): with
// two wavefronts per SIMD each has 256 registers in all, and the freed ones
// let the score products' LDS reads run ahead of the products.
template <int D>
constexpr bool kKvInLds = D == 128;

// k-steps by which the LDS reads of S and dP run ahead of their products
constexpr int kScoreReadLead = 2;

// S = Q K^T and dP = dO V^T for the wavefront's 32 keys and the 32 query
// rows 32qh.. of the tile, the keys' K and V rows read from LDS (stored like
// a streamed tile, rows own_row0..): the two products alternate k-steps, and
// each k-step's four reads are issued kScoreReadLead k-steps early.
template <typename E, int D>
__device__ __forceinline__ void scores_from_lds(const unsigned short* __restrict__ tq,
                                                const unsigned short* __restrict__ to,
                                                const unsigned short* __restrict__ kk,
                                                const unsigned short* __restrict__ vk, int own_row0, int qh,
                                                int l32, int hh, f32x16& s, f32x16& dp, const f32x16& dp0) {
  constexpr int kS = Shape<D>::kSteps;
  s = f32x16{};
  dp = dp0;
#pragma unroll
  for (int kc = 0; kc < kS; ++kc) {
    const u32x4 aq = *(const u32x4*)(tq + row_off<D>(32 * qh + l32, 2 * kc + hh));
    const u32x4 bk = *(const u32x4*)(kk + row_off<D>(own_row0 + l32, 2 * kc + hh));
    const u32x4 ao = *(const u32x4*)(to + row_off<D>(32 * qh + l32, 2 * kc + hh));
    const u32x4 bv = *(const u32x4*)(vk + row_off<D>(own_row0 + l32, 2 * kc + hh));
    s = E::mma(aq, bk, s);
    dp = E::mma(ao, bv, dp);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4 * kScoreReadLead, 0);  // LDS read
#pragma unroll
  for (int kc = 0; kc < kS; ++kc) {
    if (kc + kScoreReadLead < kS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                // MFMA
  }
}

template <typename E, int D, bool kPacked>
__global__ void __launch_bounds__(kWaveSize * kDkvWaves<D>, kDkvWavesPerSimd<D>) bwd_dkdv_kernel(BwdParams p) {
  constexpr int kW = kDkvWaves<D>, kG = kDkvGroups<D>, kKB = kDkvBlock<D>;
  using S = Shape<D, kW>;
  // Q and dO tiles (double-buffered) in one array: at the end its space holds
  // the partial sums exchanged between the two query halves
  __shared__ __attribute__((aligned(16))) unsigned short sT[2][2][kTile * D];
  unsigned short(*sQ)[kTile * D] = sT[0];
  unsigned short(*sO)[kTile * D] = sT[1];  // dO tiles
  __shared__ __attribute__((aligned(16))) float sL[2][kTile];               // lse * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[2][kTile];               // D
  __shared__ __attribute__((aligned(16))) unsigned short sKk[kKvInLds<D> ? kKB * D : 8];  // K rows of the block
  __shared__ __attribute__((aligned(16))) unsigned short sVk[kKvInLds<D> ? kKB * D : 8];  // V rows of the block

  const int tid = threadIdx.x;
  const int lane = tid & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWaveSize);
  const int kg = wave % kG;  // key group
  const int qh = wave / kG;  // query half of each tile
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4, gi = lane & 15;
  const int row_lane = 4 * hh + (gi >> 2), col_lane = 16 * (g16 & 1) + 4 * (gi & 3);

  // work item: heavy first (with a causal mask the first key blocks see the most queries)
  int bk, kb;
  if constexpr (kPacked) {
    // sequences of different lengths cost very different amounts: XCD x
    // (workgroup id mod 8) takes the (sequence, key/value head) groups x,
    // x + 8, ..., each with all its key blocks, heaviest first; the grid
    // holds 8 * ceil(groups / 8) groups and the missing ones return at once
    const int r = blockIdx.x / 8;
    const int j = r / p.n_kblocks;
    kb = r - j * p.n_kblocks;
    bk = 8 * j + blockIdx.x % 8;
    if (bk >= p.B * p.Hkv) return;
  } else {
    const int L = xcd_slice_index(blockIdx.x, p.items_dkv);
    bk = L / p.n_kblocks;
    kb = L - bk * p.n_kblocks;
  }
  const int b = bk / p.Hkv;
  const int hk = bk - b * p.Hkv;
  const SeqRows sr = seq_rows<kPacked>(p, b);
  const int Nq = sr.Nq, Nk = sr.Nk, shift = sr.shift;
  const int k0 = kb * kKB;
  if (k0 >= Nk) return;  // the whole workgroup: past this sequence's keys
  const int kw0 = k0 + kg * kRows;
  const int myk = kw0 + l32;
  // element offset of this head's key row 0 and of its query heads' row 0,
  // and the row strides (in elements) of K/V and of Q/dO
  const int kv_rs = kPacked ? p.Hkv * D : D;
  const int q_rs = kPacked ? p.Hq * D : D;
  const long long kv_head =
      kPacked ? ((long long)sr.ka * p.Hkv + hk) * D : ((long long)b * p.Hkv + hk) * (long long)Nk * D;

  u32x4 kf[kKvInLds<D> ? 1 : S::kSteps], vf[kKvInLds<D> ? 1 : S::kSteps];
  if (!kKvInLds<D>) {
    load_own_row<D>((const unsigned short*)p.k + kv_head + (long long)myk * kv_rs, myk < Nk, hh, kf);
    load_own_row<D>((const unsigned short*)p.v + kv_head + (long long)myk * kv_rs, myk < Nk, hh, vf);
  }
  f32x16 dk[S::kOutTiles], dv[S::kOutTiles];
#pragma unroll
  for (int ct = 0; ct < S::kOutTiles; ++ct) dk[ct] = dv[ct] = f32x16{};

  // queries that see some key of the block (query i stands at key position
  // i + shift): causal from key k0 on, a window up to the last key +
  // window_left
  const int wl = p.window_left;
  const int k_last = min(Nk - 1, k0 + kKB - 1);
  const int q_lo = p.causal ? max(0, k0 - shift) : 0;
  const int q_hi = wl >= 0 ? min(Nq - 1, k_last + wl - shift) : Nq - 1;
  const int t_lo = q_lo / kTile;
  const int n_t = q_hi >= q_lo ? q_hi / kTile - t_lo + 1 : 0;
  const int n_tiles = p.group * n_t;  // (query head in group, query tile)

  // visible queries of this lane's key form [vq_lo, vq_lo + vq_span]
  int vq_lo = 0x3fffffff;
  unsigned vq_span = 0u;
  if (myk < Nk) {
    const int lo = p.causal ? max(0, myk - shift) : 0;
    const int hi = wl >= 0 ? min(Nq - 1, myk + wl - shift) : Nq - 1;
    if (hi >= lo) {
      vq_lo = lo;
      vq_span = (unsigned)(hi - lo);
    }
  }
  const int wk_last = min(Nk - 1, kw0 + kRows - 1);

  CopyOffsets<D, kW> co;  // Q and dO rows
  co.init(wave, lane, 2 * q_rs);
  CopyOffsets<D, kW> ck;  // K and V rows
  ck.init(wave, lane, 2 * kv_rs);
  const int q_bytes = Nq > 0 ? (Nq - 1) * 2 * q_rs + S::kRowBytes : 0;
  const int kv_bytes = (Nk - 1) * 2 * kv_rs + S::kRowBytes;
  auto issue = [&](int tau, int buf) {
    const int g = tau / n_t;
    const int q0 = (t_lo + tau - g * n_t) * kTile;
    const long long hq = (long long)hk * p.group + g;
    const long long qh0 = kPacked ? ((long long)sr.qa * p.Hq + hq) * D : ((long long)b * p.Hq + hq) * Nq * D;
    const long long vh0 = kPacked ? hq * p.total_q + sr.qa : ((long long)b * p.Hq + hq) * Nq;
    copy_tile<D, kW>(head_rsrc(p.q, 2 * qh0, q_bytes), co, sQ[buf], q0, wave);
    copy_tile<D, kW>(head_rsrc(p.dout, 2 * qh0, q_bytes), co, sO[buf], q0, wave);
    if (wave == 0) copy_vec(head_rsrc(p.lse2, 4 * vh0, 4 * Nq), sL[buf], q0, lane);
    if (wave == 1) copy_vec(head_rsrc(p.delta, 4 * vh0, 4 * Nq), sD[buf], q0, lane);
  };

  if (kKvInLds<D>) {  // rows k0 .. k0+127 of K and V (zeros past the end)
#pragma unroll
    for (int part = 0; part < kKB / kTile; ++part) {
      copy_tile<D, kW>(head_rsrc(p.k, 2 * kv_head, kv_bytes), ck, sKk + part * kTile * D,
                              k0 + part * kTile, wave);
      copy_tile<D, kW>(head_rsrc(p.v, 2 * kv_head, kv_bytes), ck, sVk + part * kTile * D,
                              k0 + part * kTile, wave);
    }
  }
  if (n_tiles > 0) issue(0, 0);
  barrier_all();
  const float c = p.scale_log2;
  for (int tau = 0; tau < n_tiles; ++tau) {
    const int buf = tau & 1;
    if (tau + 1 < n_tiles) issue(tau + 1, buf ^ 1);
    const int g = tau / n_t;
    const int qs = (t_lo + tau - g * n_t) * kTile + 32 * qh;  // first query of this wave's half
    // skip the half when no (query, key) pair of this wavefront is visible
    const bool any = kw0 < Nk && qs < Nq && !(p.causal && qs + 31 + shift < kw0) &&
                     !(wl >= 0 && qs + shift > wk_last + wl);
    if (any) {
      const bool need_mask = qs + 32 > Nq || kw0 + kRows > Nk || (p.causal && qs + shift < kw0 + kRows - 1) ||
                             (wl >= 0 && qs + 31 + shift > kw0 + wl);
      // the dP accumulators start from -D of their rows, so they come out
      // as dP - D (element 4m+e is query row 8m + 4hh + e of the half)
      f32x16 s, dp, dp0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float4 nd = *(const float4*)(&sD[buf][32 * qh + 8 * m + 4 * hh]);
        dp0[4 * m] = nd.x;
        dp0[4 * m + 1] = nd.y;
        dp0[4 * m + 2] = nd.z;
        dp0[4 * m + 3] = nd.w;
      }
      if constexpr (kKvInLds<D>) {
        scores_from_lds<E, D>(sQ[buf], sO[buf], sKk, sVk, kg * kRows, qh, l32, hh, s, dp, dp0);
      } else {
        s = rows_times_own<E, D>(sQ[buf], qh, l32, hh, kf);
        dp = rows_times_own<E, D>(sO[buf], qh, l32, hh, vf, dp0);
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 32 * qh + 8 * m + 4 * hh;  // tile row of elements 4m .. 4m+3
        const float4 l2 = *(const float4*)(&sL[buf][r]);
        const float l2v[4] = {l2.x, l2.y, l2.z, l2.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * m + e;
          pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -l2v[e]));
          dsv[i] = pv[i] * dp[i];
        }
      }
      if (need_mask) {
        const int r0 = qs - 32 * qh;  // tile's first query
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = r0 + 32 * qh + 8 * (i >> 2) + 4 * hh + (i & 3);
          const bool vis = (unsigned)(q - vq_lo) <= vq_span;
          pv[i] = vis ? pv[i] : 0.f;
          dsv[i] = vis ? dsv[i] : 0.f;
        }
      }
      u32x4 pf[2], df[2];
      pack_operands<E>(pv, pf);
      pack_operands<E>(dsv, df);
#pragma unroll
      for (int ct = 0; ct < S::kOutTiles; ++ct) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          dv[ct] = E::mma(tr_operand<D>(sO[buf], 2 * qh + j, ct, row_lane, col_lane), pf[j], dv[ct]);
          dk[ct] = E::mma(tr_operand<D>(sQ[buf], 2 * qh + j, ct, row_lane, col_lane), df[j], dk[ct]);
        }
      }
    }
    barrier_all();
  }

  // sum the two halves' partials: the second query half's wavefronts hand
  // theirs to the first half's through the (now idle) tile buffers, one
  // tensor at a time; element 4x+y of lane l of key group kg sits at float
  // (((kg*U + x)*64 + l)*4 + y), U = 4*kOutTiles, so 16-byte accesses of a
  // wave hit consecutive addresses
  constexpr int U = 4 * S::kOutTiles;
  static_assert(sizeof(sT) >= kG * U * kWaveSize * 16, "partials must fit the tile buffers");
  float* part = reinterpret_cast<float*>(&sT[0][0][0]);
  auto exchange = [&](f32x16* acc) {
    if (qh == 1) {
#pragma unroll
      for (int ct = 0; ct < S::kOutTiles; ++ct)
#pragma unroll
        for (int x = 0; x < 4; ++x)
          *(float4*)(part + (((kg * U + 4 * ct + x) * kWaveSize + lane) << 2)) =
              float4{acc[ct][4 * x], acc[ct][4 * x + 1], acc[ct][4 * x + 2], acc[ct][4 * x + 3]};
    }
    barrier_all();
    if (qh == 0) {
#pragma unroll
      for (int ct = 0; ct < S::kOutTiles; ++ct)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float4 o = *(const float4*)(part + (((kg * U + 4 * ct + x) * kWaveSize + lane) << 2));
          acc[ct][4 * x] += o.x;
          acc[ct][4 * x + 1] += o.y;
          acc[ct][4 * x + 2] += o.z;
          acc[ct][4 * x + 3] += o.w;
        }
    }
    barrier_all();
  };
  exchange(dk);
  exchange(dv);
  if (qh == 0 && myk < Nk) {
    store_row<E, D>((unsigned short*)p.dk + kv_head + (long long)myk * kv_rs, dk, p.scale, hh);
    store_row<E, D>((unsigned short*)p.dv + kv_head + (long long)myk * kv_rs, dv, 1.f, hh);
  }
}

// ---------------------------------------------------------------------------
// 3. dQ: workgroup = (batch, query head, 128 queries), as in the forward.

template <typename E, int D, bool kPacked>
__global__ void __launch_bounds__(kThreads, 2) bwd_dq_kernel(BwdParams p) {
  using S = Shape<D>;
  __shared__ __attribute__((aligned(16))) unsigned short sK[2][kTile * D];
  __shared__ __attribute__((aligned(16))) unsigned short sV[2][kTile * D];

  const int tid = threadIdx.x;
  const int lane = tid & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWaveSize);
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4, gi = lane & 15;
  const int row_lane = 4 * hh + (gi >> 2), col_lane = 16 * (g16 & 1) + 4 * (gi & 3);

  // work item: the forward's order (causal: last query block first);
  // packed sequences deal the (sequence, key/value head) groups round-robin
  // over the XCDs as in the dK/dV kernel
  const int per_group = p.group * p.n_blocks;
  int gidx, w;
  if constexpr (kPacked) {
    const int r = blockIdx.x / 8;
    const int j = r / per_group;
    w = r - j * per_group;
    gidx = 8 * j + blockIdx.x % 8;
    if (gidx >= p.B * p.Hkv) return;
  } else {
    const int L = xcd_slice_index(blockIdx.x, p.items_dq);
    gidx = L / per_group;
    w = L - gidx * per_group;
  }
  const int qrank = w / p.group;
  const int hg = w - qrank * p.group;
  const int b = gidx / p.Hkv;
  const int hk = gidx - b * p.Hkv;
  const long long hq = (long long)hk * p.group + hg;
  const int qb = p.causal ? (p.n_blocks - 1 - qrank) : qrank;
  const SeqRows sr = seq_rows<kPacked>(p, b);
  const int Nq = sr.Nq, Nk = sr.Nk, shift = sr.shift;
  const int q0 = qb * kBlock;
  if (q0 >= Nq) return;  // the whole workgroup: past this sequence's rows
  const int wq0 = q0 + wave * kRows;
  const int myq = wq0 + l32;
  // element offsets of this head's row 0, row strides in elements, and the
  // offset of its row terms
  const int q_rs = kPacked ? p.Hq * D : D;
  const int kv_rs = kPacked ? p.Hkv * D : D;
  const long long q_head = kPacked ? ((long long)sr.qa * p.Hq + hq) * D : ((long long)b * p.Hq + hq) * Nq * D;
  const long long kv_head =
      kPacked ? ((long long)sr.ka * p.Hkv + hk) * D : ((long long)b * p.Hkv + hk) * (long long)Nk * D;
  const long long vec0 = kPacked ? hq * p.total_q + sr.qa : ((long long)b * p.Hq + hq) * Nq;

  u32x4 qf[S::kSteps], of[S::kSteps];
  load_own_row<D>((const unsigned short*)p.q + q_head + (long long)myq * q_rs, myq < Nq, hh, qf);
  load_own_row<D>((const unsigned short*)p.dout + q_head + (long long)myq * q_rs, myq < Nq, hh, of);
  const float l2 = myq < Nq ? p.lse2[vec0 + myq] : INFINITY;  // rows past the end: P = 0
  const float nd = myq < Nq ? p.delta[vec0 + myq] : 0.f;  // -D
  f32x16 dq[S::kOutTiles];
#pragma unroll
  for (int ct = 0; ct < S::kOutTiles; ++ct) dq[ct] = f32x16{};

  // key tiles this workgroup needs (query i stands at key position
  // i + shift), and this lane's visible keys [vis_lo, vis_lo + vis_span]
  const int wl = p.window_left;
  const int kend = p.causal ? min(Nk, q0 + kBlock + shift) : Nk;
  const int kbeg = wl >= 0 ? max(0, q0 + shift - wl) : 0;
  const int t_beg = kbeg / kTile, t_end = kend > kbeg ? (kend + kTile - 1) / kTile : t_beg;
  int vis_lo = 0x3fffffff;
  unsigned vis_span = 0u;
  if (myq < Nq) {
    const int pos = myq + shift;
    const int lo = wl >= 0 ? max(0, pos - wl) : 0;
    const int hi = p.causal ? min(pos, Nk - 1) : Nk - 1;
    if (hi >= lo) {
      vis_lo = lo;
      vis_span = (unsigned)(hi - lo);
    }
  }
  const int wq1 = min(Nq, wq0 + kRows) - 1;

  CopyOffsets<D> co;
  co.init(wave, lane, 2 * kv_rs);
  const int kv_bytes = Nk > 0 ? (Nk - 1) * 2 * kv_rs + S::kRowBytes : 0;
  auto issue = [&](int t, int buf) {
    copy_tile<D>(head_rsrc(p.k, 2 * kv_head, kv_bytes), co, sK[buf], t * kTile, wave);
    copy_tile<D>(head_rsrc(p.v, 2 * kv_head, kv_bytes), co, sV[buf], t * kTile, wave);
  };

  if (t_beg < t_end) issue(t_beg, 0);
  barrier_all();
  for (int t = t_beg; t < t_end; ++t) {
    const int buf = (t - t_beg) & 1;
    if (t + 1 < t_end) issue(t + 1, buf ^ 1);
    const int kb = t * kTile;
    const bool any = wq0 < Nq && !(p.causal && kb > wq1 + shift) && !(wl >= 0 && kb + kTile - 1 < wq0 + shift - wl);
    if (any) {
      const bool need_mask = kb + kTile > Nk || (p.causal && kb + kTile - 1 > wq0 + shift) ||
                             (wl >= 0 && kb < wq1 + shift - wl);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x16 s = rows_times_own<E, D>(sK[buf], h, l32, hh, qf);   // S^T[key][query]
        f32x16 dp0;  // -D of the lane's query: the accumulators come out as dP - D
#pragma unroll
        for (int i = 0; i < 16; ++i) dp0[i] = nd;
        const f32x16 dp = rows_times_own<E, D>(sV[buf], h, l32, hh, of, dp0);  // (dP - D)^T[key][query]
        float dsv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          dsv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.scale_log2, -l2)) * dp[i];
        // one branch around the whole block (a test per element would be
        // turned into selects that every tile pays for)
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb + 32 * h + 8 * (i >> 2) + 4 * hh + (i & 3);
            dsv[i] = (unsigned)(key - vis_lo) <= vis_span ? dsv[i] : 0.f;
          }
        }
        u32x4 df[2];
        pack_operands<E>(dsv, df);
#pragma unroll
        for (int ct = 0; ct < S::kOutTiles; ++ct) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            dq[ct] = E::mma(tr_operand<D>(sK[buf], 2 * h + j, ct, row_lane, col_lane), df[j], dq[ct]);
        }
      }
    }
    barrier_all();
  }
  // the output row is rebuilt from the lane index (through an empty asm
  // statement) rather than kept in registers across the key loop
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int myq_out = wq0 + (ln & 31);
  if (myq_out < Nq)
    store_row<E, D>((unsigned short*)p.dq + q_head + (long long)myq_out * q_rs, dq, p.scale, ln >> 5);
}

template <typename E, int D, bool kPacked>
hipError_t launch_t(const BwdParams& p, hipStream_t stream) {
  constexpr int kRowsPerPrepBlock = 256 / (D / 8);
  const long long prep_blocks = (p.rows + kRowsPerPrepBlock - 1) / kRowsPerPrepBlock;
  hipLaunchKernelGGL((bwd_prep_kernel<E, D, kPacked>), dim3((unsigned)prep_blocks), dim3(256), 0, stream, p);
  // packed: the grids hold 8 * ceil(groups / 8) (sequence, key/value head) groups
  const long long groups8 = 8 * (((long long)p.B * p.Hkv + 7) / 8);
  const long long g_dkv = kPacked ? groups8 * p.n_kblocks : p.items_dkv;
  const long long g_dq = kPacked ? groups8 * p.group * p.n_blocks : p.items_dq;
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, kPacked>), dim3((unsigned)g_dkv), dim3(kWaveSize * kDkvWaves<D>), 0,
                     stream, p);
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, kPacked>), dim3((unsigned)g_dq), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  BwdParams p = make_bwd_params(a, kBlock);
  // the dK/dV workgroups own kDkvBlock<D> keys each
  const int nk = a.cu_q ? a.max_k : a.N;
  p.n_kblocks = (nk + kDkvBlock<D> - 1) / kDkvBlock<D>;
  p.items_dkv = a.B * a.Hkv * p.n_kblocks;
  return a.cu_q ? launch_t<E, D, true>(p, stream) : launch_t<E, D, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch<Bf16, 64>(a, stream) : launch<Bf16, 128>(a, stream);
}

hipError_t launch_bwd_f16(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch<F16, 64>(a, stream) : launch<F16, 128>(a, stream);
}

long long bwd_rows_per_workgroup() { return kBlock; }

long long bwd_keys_per_workgroup(int d) { return d == 64 ? kDkvBlock<64> : kDkvBlock<128>; }

}  // namespace fa
