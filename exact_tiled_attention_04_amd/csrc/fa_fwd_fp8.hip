// Exact attention forward with FP8 inputs on CDNA4 matrix cores (gfx950).
//
// The FlashAttention quiz (question 6) and the FlashAttention-2 (PL) article
// (section "FlashAttention-3") name 8-bit floating point, with measures that
// keep its rounding error in check, as the next step for speed.  This kernel
// computes the attention of the 16-bit forward (scale * q.k, causal and
// left-window masks, grouped key/value heads, an online softmax over key
// tiles staged in LDS) with both products on the FP8 matrix cores:
//
//   * inputs are OCP E4M3 bytes with one float32 scale per tensor; an
//     element stands for e4m3(byte) * scale.  The score product runs on the
//     bytes; the Q and K scales fold into the exponent's multiplier
//     (scale * q_scale * k_scale * log2 e) and the V scale into the final
//     1/l, so no input is ever rescaled;
//   * error management: both products accumulate in fp32, the row sum l is
//     taken over the fp32 probabilities, and only the probability operand of
//     the second product is rounded to E4M3.  Probabilities are taken
//     relative to 2^-7 of the running reference max, so a row's largest one
//     lands in [2^7, 2^8.5] (E4M3 tops out at 448): 3 mantissa bits hold down
//     to 2^-14.5 of the row max, and only what lies below about 2^-17.5 of
//     it rounds to zero;
//   * O is written as bfloat16 and lse as float32 (natural log of the sum
//     over the dequantised scores), as in the 16-bit forward.
//
// Matrix-core mapping (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales:
// A 32x64, B 64x32, C 32x32 fp32; lane l brings 32 bytes of row l%32 of A
// and 32 bytes of column l%32 of B, for the same 32 reduction indices, chosen
// by l/32; C[8*(i/4)+4*(l/32)+i%4][l%32] for i < 16, as in the 16-bit kernel):
//
//   S^T = K Q^T     A = 32 key rows, 32 contiguous bytes each from LDS (two
//                   16-byte reads), B = this lane's query row, held in
//                   registers; one product spans 64 head dimensions.
//   O^T += V^T P^T  B = the lane's own 32 probabilities of a 64-key block,
//                   packed 4 per dword straight from the score accumulators,
//                   so reduction slot (l/32, byte p) holds key
//                   32(p/16) + 8((p%16)/4) + 4(l/32) + p%4;  A = V^T from
//                   row-major V in LDS through the 8-bit transposing LDS read
//                   (ds_read_b64_tr_b8), four reads per product, addressed
//                   so that every lane receives exactly those keys.
#include "fa_internal.h"
#include "fa_mfma_common.h"

#include <type_traits>

namespace fa {
namespace {

using namespace mfma;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaveSize * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBR = kWaves * kRowsPerWave;  // query rows per workgroup
#ifndef FA8_KEYS_PER_TILE
#define FA8_KEYS_PER_TILE 64
#endif
// Three waves per SIMD at d = 128 (a register budget of 168, met without
// spilling by rebuilding lane-derived offsets where they are used); d = 64
// needs fewer registers and reaches four either way.
#ifndef FA8_WAVES_PER_SIMD
#define FA8_WAVES_PER_SIMD 3
#endif
constexpr int kBC = FA8_KEYS_PER_TILE;  // keys per K/V tile
constexpr int kHalves = kBC / 32;       // 32-key score blocks per tile
constexpr int kBlocks64 = kBC / 64;     // 64-key probability blocks per tile
static_assert(kBC == 64 || kBC == 128, "tile width");
constexpr float kLn2 = 0.69314718055994531f;

// Probabilities are exp2(x - (m_use - kPOffset)): the reference max maps to
// 2^kPOffset.  The reference max moves only when the row max gets ahead of it
// by more than kRescaleSlack, so probabilities stay below
// 2^(kPOffset + kRescaleSlack) = 362 < 448, the largest E4M3 value.
constexpr float kPOffset = 7.0f;
constexpr float kRescaleSlack = 1.5f;

__device__ __forceinline__ f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
  // operand formats 0/0 = E4M3 for A and B; E8M0 block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
  return __builtin_shufflevector(__builtin_bit_cast(i32x4, lo), __builtin_bit_cast(i32x4, hi), 0, 1, 2, 3, 4, 5,
                                 6, 7);
}

// Four fp32 values -> four E4M3 bytes (round to nearest even), first lowest.
__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D>
struct Shape {
  static constexpr int kChunks = D / 16;     // 16-byte chunks per row
  static constexpr int kSteps = D / 64;      // score products over the head dimension
  static constexpr int kOutTiles = D / 32;   // 32-wide output channel tiles
  static constexpr int kRowBytes = D;
  // one wave-wide 16-byte-per-lane load moves 1 KiB = this many rows
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;
  static constexpr int kLoadsPerWave = kBC / kRowsPerLoad / kWaves;
  static_assert(kBC % (kRowsPerLoad * kWaves) == 0, "tile must split evenly over the wavefronts");
};

// LDS layouts.  Both tiles are row-major [key][dim] bytes; 16-byte chunks of
// a row are permuted by an XOR with a function of the row so that the reads of
// the hot loop hit distinct banks (gfx950's LDS serves 256 bytes per clock):
//   K: each 16-lane group reads one 16-byte chunk of 16 consecutive rows.
//     D=128 (two rows per 256 bytes): chunk ^ ((row / 2) mod 8);
//     D=64 (four rows per 256 bytes): chunk ^ ((row / 4) mod 4).
//   V: a transposing read covers 16 rows x 32 bytes (a 32-byte quad); each
//     half-wave takes the rows 16r + {0..3, 8..11} (+4 for the upper half).
//     The quad is XORed with a row function that separates those rows:
//     D=128: bit 1 and bit 3 of the row; D=64: bit 3.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int v_quad_swz(int row) {
  return D == 128 ? (((row >> 1) & 1) | (((row >> 3) & 1) << 1)) : ((row >> 3) & 1);
}

// Per-lane byte offsets (within one tile) of this lane's pieces of the
// direct-to-LDS copies: lane l fills LDS bytes 16l..16l+15 of its 1-KiB
// piece, so it fetches the logical chunk the swizzle maps there.
template <int D>
struct LoadOffsets {
  int k[Shape<D>::kLoadsPerWave];
  int v[Shape<D>::kLoadsPerWave];
  __device__ __forceinline__ void init(int wave, int lane) {
    using S = Shape<D>;
#pragma unroll
    for (int u = 0; u < S::kLoadsPerWave; ++u) {
      const int piece = wave * S::kLoadsPerWave + u;
      const int row = piece * S::kRowsPerLoad + lane / S::kChunks;
      const int pch = lane % S::kChunks;
      k[u] = row * S::kRowBytes + ((pch ^ k_swz<D>(row)) << 4);
      v[u] = row * S::kRowBytes + ((pch ^ (v_quad_swz<D>(row) << 1)) << 4);
    }
  }
};

// Start copying key tile t of K (or V) from device memory straight into LDS.
// Rows past the end of the sequence lie outside the buffer's range and
// arrive as zeros.
template <int D>
__device__ __forceinline__ void copy_tile_async(__amdgpu_buffer_rsrc_t r, const int* lane_off, unsigned char* dst,
                                                int t, int wave) {
  using S = Shape<D>;
  const int tile_bytes = t * (kBC * S::kRowBytes);
#pragma unroll
  for (int u = 0; u < S::kLoadsPerWave; ++u) {
    const int piece = wave * S::kLoadsPerWave + u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + piece * 1024), 16, lane_off[u], tile_bytes, 0,
                                             0);
  }
}

// The lane index through an empty asm statement: values derived from it are
// then recomputed where they are used instead of being hoisted out of the
// key loop and held in registers (or spilled) across it.
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

template <int D>
struct LoopCtx {
  __amdgpu_buffer_rsrc_t rk, rv;
  LoadOffsets<D> off;
  int N, wl, t_beg, t_end;
  int wave, lane, l32, hh;
  int wq0, wq1;
  int k_base;  // byte offset of chunk 2hh of the lane's K row (row l32 of the tile)
  // byte offset of this lane's transposing V read for output tile 0; tile ct
  // reads at v_base ^ 32 ct (the tile index occupies bits 5-6 alone)
  int v_base;
  bool causal;
  float c;                          // scale * q_scale * k_scale * log2(e)
};

template <int D>
struct RowState {
  i32x8 qf[Shape<D>::kSteps];        // q row (E4M3 bytes) as the B operand
  f32x16 oacc[Shape<D>::kOutTiles];  // unnormalised O^T columns, in units of the V bytes
  float m_use;                       // reference max (log2 units)
  float l_run;                       // running sum of this half-wave's probabilities
};

// Scores of key tile t: S^T = K Q^T; s[h] holds keys kBC*t + 32h .. +31.
// The lane reads 16-byte chunks 4kc + 2hh and 4kc + 2hh + 1 of its row; the
// three index bits are distinct, so the swizzled byte offset is
// x.k_base ^ 64 kc ^ 16 (one register kept across the loop, two XORs a step).
template <int D>
__device__ __forceinline__ void tile_scores(const unsigned char* __restrict__ cK, const LoopCtx<D>& x,
                                            const RowState<D>& st, f32x16 (&s)[kHalves]) {
#pragma unroll
  for (int h = 0; h < kHalves; ++h) s[h] = f32x16{};
  const int kbase = opaque_lane(x.k_base);
#pragma unroll
  for (int kc = 0; kc < Shape<D>::kSteps; ++kc) {
    const int a_lo = kbase ^ (64 * kc);
    const int a_hi = a_lo ^ 16;
#pragma unroll
    for (int h = 0; h < kHalves; ++h) {
      const u32x4 lo = *(const u32x4*)(cK + a_lo + 32 * h * D);
      const u32x4 hi = *(const u32x4*)(cK + a_hi + 32 * h * D);
      s[h] = mma8(join(lo, hi), st.qf[kc], s[h]);
    }
  }
}

// Mask tile t where it crosses the causal diagonal, the window edge or the
// sequence end for some row of the wavefront: key kb + off is visible iff
// 0 <= kb + off - vis_lo <= vis_span.
// The lane's visible range is rebuilt from its lane index each time (a few
// vector operations on the rare masked tiles) rather than kept in registers
// across the key loop, where three waves per SIMD leave none to spare.
template <int D>
__device__ __forceinline__ void tile_mask(const LoopCtx<D>& x, int t, f32x16 (&s)[kHalves]) {
  const int kb = t * kBC;
  const int ke = kb + kBC - 1;
  const bool need_mask = (ke >= x.N) || (x.causal && ke > x.wq0) || (x.wl >= 0 && kb < x.wq1 - x.wl);
  if (!need_mask) return;
  const int ln = opaque_lane(x.lane);
  const int myq = x.wq0 + (ln & 31);
  const int vis_lo = x.wl >= 0 ? max(0, myq - x.wl) : 0;
  const int vis_hi = x.causal ? min(myq, x.N - 1) : x.N - 1;
  const unsigned vis_span = (unsigned)(vis_hi - vis_lo);
  const int base = kb - vis_lo + 4 * (ln >> 5);
#pragma unroll
  for (int h = 0; h < kHalves; ++h) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int off = 32 * h + 8 * (i >> 2) + (i & 3);
      s[h][i] = ((unsigned)(base + off) <= vis_span) ? s[h][i] : -INFINITY;
    }
  }
}

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

// Sum of N values as a balanced tree of two-input adds (depth log2 N
// instead of a serial chain of N - 1 dependent adds).
template <int N>
__device__ __forceinline__ float sum_tree(const float* a) {
  if constexpr (N == 1) {
    return a[0];
  } else {
    return sum_tree<N / 2>(a) + sum_tree<N - N / 2>(a + N / 2);
  }
}

// Online softmax of one score tile: turns s into the E4M3 probability
// operands pf (8 dwords per 64-key block), updates the row's reference max
// and sum, and returns the factor the partial output must be multiplied by.
template <int D>
__device__ __forceinline__ float tile_softmax(const LoopCtx<D>& x, RowState<D>& st, f32x16 (&s)[kHalves],
                                              i32x8* pf) {
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
  // When bumped, mx is finite and m_use - mx finite or -inf; otherwise the
  // factor is exactly 1: no NaN can arise.
  const bool bump = mx > st.m_use + kRescaleSlack;
  const float alpha = bump ? __builtin_amdgcn_exp2f(st.m_use - mx) : 1.f;
  st.m_use = bump ? mx : st.m_use;
  const float m_exp = (st.m_use == -INFINITY) ? 0.f : st.m_use - kPOffset;
#pragma unroll
  for (int h = 0; h < kHalves; ++h) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[h][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][i], x.c, -m_exp));
      sv[16 * h + i] = s[h][i];
    }
  }
  const float rs = sum_tree<16 * kHalves>(sv);
  st.l_run = __builtin_fmaf(st.l_run, alpha, rs);
  // dword w of block b packs keys of s[2b + w/4], elements 4(w%4) .. +3
#pragma unroll
  for (int b = 0; b < kBlocks64; ++b) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const f32x16& sh = s[2 * b + w / 4];
      const int i0 = 4 * (w % 4);
      pf[b][w] = pack4_fp8(sh[i0], sh[i0 + 1], sh[i0 + 2], sh[i0 + 3]);
    }
  }
  return alpha;
}

// O^T += V^T P^T for one tile: per output tile and 64-key block, four
// transposing reads give the lane's 32 bytes of V^T (read r covers keys
// 16r .. 16r+15 of the block), then one product.
template <int D>
__device__ __forceinline__ void tile_pv(const unsigned char* __restrict__ vC, const LoopCtx<D>& x, RowState<D>& st,
                                        const i32x8* pf) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
#pragma unroll
  for (int ct = 0; ct < Shape<D>::kOutTiles; ++ct) {
#pragma unroll
    for (int b = 0; b < kBlocks64; ++b) {
      i32x2 r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        r[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2*)(vC + (x.v_base ^ (32 * ct)) + (64 * b + 16 * q) * D));
      const i32x8 a = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
      st.oacc[ct] = mma8(a, pf[b], st.oacc[ct]);
    }
  }
}

__device__ __forceinline__ void rescale_if_needed(float alpha, f32x16* oacc, int tiles) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
    for (int ct = 0; ct < tiles; ++ct) oacc[ct] *= alpha;
  }
}

// One step of the key loop, pipelined as in the 16-bit kernel: scores of
// tile t on the matrix cores at raised priority, then the softmax of tile t
// interleaved with O += P(t-1) V(t-1).  K travels two tiles ahead, V one.
template <int D, bool kHasPrev>
__device__ __forceinline__ void pipeline_step(const unsigned char* __restrict__ kC, unsigned char* __restrict__ kN,
                                              const unsigned char* __restrict__ vC, unsigned char* __restrict__ vN,
                                              const LoopCtx<D>& x, RowState<D>& st, i32x8* pf_prev,
                                              float& alpha_prev, int t) {
  using S = Shape<D>;
  copy_tile_async<D>(x.rv, x.off.v, vN, t, x.wave);
  copy_tile_async<D>(x.rk, x.off.k, kN, t + 2, x.wave);

  f32x16 s[kHalves];
  __builtin_amdgcn_s_setprio(2);
  tile_scores<D>(kC, x, st, s);
  __builtin_amdgcn_s_setprio(0);
  tile_mask<D>(x, t, s);

  if (kHasPrev) rescale_if_needed(alpha_prev, st.oacc, S::kOutTiles);

  i32x8 pf[kBlocks64];
  const float alpha = tile_softmax<D>(x, st, s, pf);
  if (kHasPrev) {
    tile_pv<D>(vC, x, st, pf_prev);
    // each PV product follows a small slice of the softmax work (eight
    // vector operations per 64-key block: of 8 to 40 measured, the fastest);
    // its four reads were issued one product earlier
    constexpr int kPv = kBlocks64 * S::kOutTiles;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS read
#pragma unroll
    for (int g = 0; g < kPv; ++g) {
      if (g + 1 < kPv) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 8 / kBlocks64, 0);       // VALU
    }
  }
#pragma unroll
  for (int j = 0; j < kBlocks64; ++j) pf_prev[j] = pf[j];
  alpha_prev = alpha;
}

template <int kInFlight>
__device__ __forceinline__ void tile_barrier() {
  static_assert(kInFlight >= 0 && kInFlight < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kInFlight) : "memory");
}

template <int D>
__global__ void __launch_bounds__(kThreads, FA8_WAVES_PER_SIMD) fwd_fp8_kernel(FwdParams p) {
  using S = Shape<D>;
  __shared__ __attribute__((aligned(16))) unsigned char sK0[kBC * D];
  __shared__ __attribute__((aligned(16))) unsigned char sK1[kBC * D];
  __shared__ __attribute__((aligned(16))) unsigned char sK2[kBC * D];
  __shared__ __attribute__((aligned(16))) unsigned char sV0[kBC * D];
  __shared__ __attribute__((aligned(16))) unsigned char sV1[kBC * D];

  LoopCtx<D> x;
  const int tid = threadIdx.x;
  x.lane = tid & (kWaveSize - 1);
  x.wave = __builtin_amdgcn_readfirstlane(tid / kWaveSize);
  x.l32 = x.lane & 31;
  x.hh = x.lane >> 5;
  x.off.init(x.wave, x.lane);
  x.k_base = x.l32 * D + (((2 * x.hh) ^ k_swz<D>(x.l32)) << 4);

  const WorkItem it = decode_work_item(p, blockIdx.x);
  const int N = p.N;
  x.N = N;
  const int b = it.bh / p.Hq;
  const int hq = it.bh - b * p.Hq;
  const int hk = hq / p.group;
  const long long q_head = (long long)it.bh * N * D;
  const long long kv_head = ((long long)b * p.Hkv + hk) * N * D;
  const unsigned char* __restrict__ qg = (const unsigned char*)p.q + q_head;
  const int head_bytes = N * S::kRowBytes;
  x.rk = __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)p.k + kv_head), 0, head_bytes,
                                           kBufferFlags);
  x.rv = __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)p.v + kv_head), 0, head_bytes,
                                           kBufferFlags);

  x.causal = p.causal != 0;
  x.wl = p.window_left;
  x.c = p.scale_log2;
  const int q0 = it.qb * kBR;
  x.wq0 = q0 + x.wave * kRowsPerWave;
  x.wq1 = min(N, x.wq0 + kRowsPerWave) - 1;
  const int myq = x.wq0 + x.l32;

  const int kend = x.causal ? min(N, q0 + kBR) : N;
  const int kbeg = x.wl >= 0 ? max(0, q0 - x.wl) : 0;
  x.t_beg = kbeg / kBC;
  x.t_end = (kend + kBC - 1) / kBC;


  // Transposing V read: in each 16-lane group G, lane s = 2e + j supplies the
  // address for byte e of the group's outputs (key row 8(e/4) + 4(G/2) + e%4
  // of a 16-row slab) and for columns 16(G%2) + 8j .. +7 of the 32-byte quad.
  {
    const int s16 = x.lane & 15;
    const int e = s16 >> 1, j = s16 & 1, g = x.lane >> 4;
    const int row = 8 * (e >> 2) + 4 * (g >> 1) + (e & 3);
    const int f = v_quad_swz<D>(row);  // the same for every 16-row slab
    x.v_base = row * D + 32 * f + 16 * (g & 1) + 8 * j;
  }

  RowState<D> st;
#pragma unroll
  for (int kc = 0; kc < S::kSteps; ++kc) {
    if (myq < N) {
      const unsigned char* src = qg + (long long)myq * D + 64 * kc + 32 * x.hh;
      st.qf[kc] = join(q_signed8(*(const u32x4*)src, p.q_sign), q_signed8(*(const u32x4*)(src + 16), p.q_sign));
    } else {
      st.qf[kc] = i32x8{};
    }
  }
#pragma unroll
  for (int ct = 0; ct < S::kOutTiles; ++ct) st.oacc[ct] = f32x16{};
  st.m_use = -INFINITY;
  st.l_run = 0.f;

  auto kbuf = [&](int j) { return j == 0 ? sK0 : (j == 1 ? sK1 : sK2); };
  auto vbuf = [&](int j) { return j == 0 ? sV0 : sV1; };
  constexpr int kInFlight = S::kLoadsPerWave;  // the previous step's K copy
  const int t0 = x.t_beg;
  copy_tile_async<D>(x.rk, x.off.k, sK0, t0, x.wave);
  copy_tile_async<D>(x.rk, x.off.k, sK1, t0 + 1, x.wave);  // past the end: zeros, never read
  i32x8 pf_prev[kBlocks64];
  float alpha_prev = 1.f;
  tile_barrier<0>();
  pipeline_step<D, false>(sK0, sK2, sV1, sV0, x, st, pf_prev, alpha_prev, t0);
  auto step = [&](auto uc, int t) {
    constexpr int u = decltype(uc)::value;  // (t - t0) % 6
    tile_barrier<kInFlight>();
    pipeline_step<D, true>(kbuf(u % 3), kbuf((u + 2) % 3), vbuf((u + 1) % 2), vbuf(u % 2), x, st, pf_prev,
                           alpha_prev, t);
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
  if ((x.t_end - 1 - t0) % 2 == 0)
    tile_pv<D>(sV0, x, st, pf_prev);
  else
    tile_pv<D>(sV1, x, st, pf_prev);

  float llo, lhi;
  half_pair(st.l_run, llo, lhi);
  const float l_tot = llo + lhi;
  const int ln = opaque_lane(x.lane);
  const int hh = ln >> 5;
  const int myq_out = x.wq0 + (ln & 31);
  if (myq_out < N) {
    const float inv = p.o_mult / l_tot;
    unsigned short* og = (unsigned short*)p.o + q_head + (long long)myq_out * D;
#pragma unroll
    for (int ct = 0; ct < S::kOutTiles; ++ct) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const u32x2 w = u32x2{Bf16::pack2(st.oacc[ct][4 * gq + 0] * inv, st.oacc[ct][4 * gq + 1] * inv),
                              Bf16::pack2(st.oacc[ct][4 * gq + 2] * inv, st.oacc[ct][4 * gq + 3] * inv)};
        *(u32x2*)(og + 32 * ct + 8 * gq + 4 * hh) = w;
      }
    }
    if (hh == 0 && p.lse != nullptr)
      p.lse[(long long)it.bh * N + myq_out] = (st.m_use - kPOffset + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

template <int D>
hipError_t launch(const FwdArgs& a, float q_scale, float k_scale, float v_scale, hipStream_t stream) {
  FwdParams p = make_params(a, kBR);  // q_sign from the sign of the scale (the Q and K scales are > 0)
  const double c = (double)a.scale * q_scale * k_scale;
  p.scale_log2 = (float)((c != 0.0 ? (c < 0.0 ? -c : c) : 1.0) * 1.4426950408889634);
  p.o_mult = v_scale;
  hipLaunchKernelGGL((fwd_fp8_kernel<D>), dim3(p.total_items), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdArgs& a, float q_scale, float k_scale, float v_scale, hipStream_t stream) {
  return a.d == 64 ? launch<64>(a, q_scale, k_scale, v_scale, stream)
                   : launch<128>(a, q_scale, k_scale, v_scale, stream);
}

long long fp8_rows_per_workgroup() { return kBR; }

}  // namespace fa
