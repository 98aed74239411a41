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

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaveSize = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaveSize * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBR = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBC = 64;                     // keys per K/V tile
constexpr float kLn2 = 0.69314718055994531f;

struct Bf16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two floats -> two bf16 (round to nearest even) in one dword, low first
  static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(unsigned, v);
  }
};

struct F16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(unsigned, v);
  }
};

template <int D>
struct Shape {
  static constexpr int kChunks = D / 8;    // 16-byte chunks per row
  static constexpr int kSteps = D / 16;    // MFMA k-steps over the head dimension
  static constexpr int kOutTiles = D / 32; // 32-wide output channel tiles
  static constexpr int kChunksPerThread = kBC * kChunks / kThreads;
  static_assert(kBC * kChunks % kThreads == 0, "tile must split evenly over the workgroup");
};

// LDS layouts.  Both tiles are row-major [key][dim] with 16-byte chunks
// permuted within a row by an XOR of the row index:
//   K: chunk ^ (row mod chunks-per-row).  A K read has the 32 lanes of a half
//      wave on 32 consecutive rows at one logical chunk; the XOR spreads any
//      16 consecutive rows over all chunk positions (all banks).
//   V: chunk ^ 2*(row mod 4).  A transposing read has each 16-lane group on 4
//      consecutive rows x 32 bytes; the XOR puts those 4 rows' 32-byte pieces
//      in distinct banks.
template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * D + ((chunk ^ (row & (Shape<D>::kChunks - 1))) << 3);
}
template <int D>
__device__ __forceinline__ int v_off(int row, int col) {
  return row * D + ((((col >> 3) ^ ((row & 3) << 1))) << 3) + (col & 7);
}

// Exchange with the lane 32 away: returns the pair in a fixed order (lower
// half-wave's value first) so both lanes compute bit-identical results.
__device__ __forceinline__ void half_pair(float x, float& lo, float& hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

__device__ __forceinline__ s16x4 lds_read_tr(const unsigned short* base, int off) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
}

template <typename E, int D>
__global__ void __launch_bounds__(kThreads, 2) fwd_mfma_kernel(FwdParams p) {
  using S = Shape<D>;
  __shared__ __attribute__((aligned(16))) unsigned short sK[kBC * D];
  __shared__ __attribute__((aligned(16))) unsigned short sV[kBC * D];

  const int tid = threadIdx.x;
  const int lane = tid & (kWaveSize - 1);
  const int wave = tid / kWaveSize;
  const int l32 = lane & 31;
  const int hh = lane >> 5;  // which half-wave

  const WorkItem it = decode_work_item(p, blockIdx.x);
  const int N = p.N;
  const int b = it.bh / p.Hq;
  const int hq = it.bh - b * p.Hq;
  const int hk = hq / p.group;
  const long long q_head = (long long)it.bh * N * D;
  const long long kv_head = ((long long)b * p.Hkv + hk) * N * D;
  const unsigned short* __restrict__ qg = (const unsigned short*)p.q + q_head;
  const unsigned short* __restrict__ kg = (const unsigned short*)p.k + kv_head;
  const unsigned short* __restrict__ vg = (const unsigned short*)p.v + kv_head;

  const bool causal = p.causal != 0;
  const int wl = p.window_left;
  const int q0 = it.qb * kBR;
  const int wq0 = q0 + wave * kRowsPerWave;          // first row of this wavefront
  const int wq1 = min(N, wq0 + kRowsPerWave) - 1;    // last valid row (< wq0 if none)
  const int myq = wq0 + l32;                         // this lane's query row

  // Key tiles this workgroup needs: causal stops at its last row, a window
  // starts window_left keys before its first row.
  const int kend = causal ? min(N, q0 + kBR) : N;
  const int kbeg = wl >= 0 ? max(0, q0 - wl) : 0;
  const int t_beg = kbeg / kBC;
  const int t_end = (kend + kBC - 1) / kBC;

  // Q as the B operand: q[myq][16*kc + 8*hh .. +7] for each k-step kc.
  u32x4 qf[S::kSteps];
#pragma unroll
  for (int kc = 0; kc < S::kSteps; ++kc) {
    if (myq < N)
      qf[kc] = *(const u32x4*)(qg + (long long)myq * D + 16 * kc + 8 * hh);
    else
      qf[kc] = u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 oacc[S::kOutTiles];
#pragma unroll
  for (int ct = 0; ct < S::kOutTiles; ++ct) oacc[ct] = f32x16{};
  float m_run = -INFINITY;  // running max of scale*log2(e)*score
  float l_run = 0.f;        // running sum of exp2(... - m_run) over this half-wave's keys
  const float c = p.scale_log2;

  // Global -> register staging of one K/V tile (zero rows past the end).
  u32x4 kreg[S::kChunksPerThread], vreg[S::kChunksPerThread];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < S::kChunksPerThread; ++u) {
      const int ci = tid + u * kThreads;
      const int row = ci / S::kChunks;
      const int ch = ci % S::kChunks;
      const int key = t * kBC + row;
      if (key < N) {
        kreg[u] = *(const u32x4*)(kg + (long long)key * D + ch * 8);
        vreg[u] = *(const u32x4*)(vg + (long long)key * D + ch * 8);
      } else {
        kreg[u] = u32x4{0u, 0u, 0u, 0u};
        vreg[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < S::kChunksPerThread; ++u) {
      const int ci = tid + u * kThreads;
      const int row = ci / S::kChunks;
      const int ch = ci % S::kChunks;
      *(u32x4*)(sK + k_off<D>(row, ch)) = kreg[u];
      *(u32x4*)(sV + v_off<D>(row, ch * 8)) = vreg[u];
    }
  };

  // Lane geometry of the transposing V read (see the header comment).
  const int g16 = lane >> 4;
  const int gi = lane & 15;
  const int v_row_lane = 4 * hh + (gi >> 2);
  const int v_col_lane = 16 * (g16 & 1) + 4 * (gi & 3);

  if (t_beg < t_end) load_tile(t_beg);
  for (int t = t_beg; t < t_end; ++t) {
    __syncthreads();  // every wavefront is done with the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < t_end) load_tile(t + 1);  // in flight while this tile computes

    const int kb = t * kBC;
    const int ke = kb + kBC - 1;
    const bool skip = (wq0 >= N) || (causal && kb > wq1) || (wl >= 0 && ke < wq0 - wl);
    if (skip) continue;
    const bool need_mask = (ke >= N) || (causal && ke > wq0) || (wl >= 0 && kb < wq1 - wl);

    // ---- scores: S^T = K Q^T, keys kb..kb+31 in s0 and kb+32..kb+63 in s1
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int kc = 0; kc < S::kSteps; ++kc) {
      const u32x4 a0 = *(const u32x4*)(sK + k_off<D>(l32, 2 * kc + hh));
      const u32x4 a1 = *(const u32x4*)(sK + k_off<D>(32 + l32, 2 * kc + hh));
      s0 = E::mma(a0, qf[kc], s0);
      s1 = E::mma(a1, qf[kc], s1);
    }

    // ---- mask: only on tiles that cross the causal diagonal, the window
    // edge or the end of the sequence
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb + 8 * (i >> 2) + 4 * hh + (i & 3);
        const bool h0 = key >= N || (causal && key > myq) || (wl >= 0 && key < myq - wl);
        const bool h1 = key + 32 >= N || (causal && key + 32 > myq) || (wl >= 0 && key + 32 < myq - wl);
        s0[i] = h0 ? -INFINITY : s0[i];
        s1[i] = h1 ? -INFINITY : s1[i];
      }
    }

    // ---- online softmax (base 2, scale folded into the exponent)
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    float mlo, mhi;
    half_pair(mx, mlo, mhi);
    mx = fmaxf(mlo, mhi);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // nothing visible yet
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -m_use));
      s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -m_use));
      rs += s0[i] + s1[i];
    }
    l_run = l_run * alpha + rs;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int ct = 0; ct < S::kOutTiles; ++ct) oacc[ct] *= alpha;
    }

    // ---- P^T operands: the lane's own probabilities, 8 keys per k-step
    u32x4 pf[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      pf[j] = u32x4{E::pack2(s0[8 * j + 0], s0[8 * j + 1]), E::pack2(s0[8 * j + 2], s0[8 * j + 3]),
                    E::pack2(s0[8 * j + 4], s0[8 * j + 5]), E::pack2(s0[8 * j + 6], s0[8 * j + 7])};
      pf[2 + j] = u32x4{E::pack2(s1[8 * j + 0], s1[8 * j + 1]), E::pack2(s1[8 * j + 2], s1[8 * j + 3]),
                        E::pack2(s1[8 * j + 4], s1[8 * j + 5]), E::pack2(s1[8 * j + 6], s1[8 * j + 7])};
    }

    // ---- O^T += V^T P^T.  k-step mc covers keys 16mc..16mc+15 in the order
    // the accumulator hands them over: half-wave hh holds keys
    // 16mc + 4hh + {0..3} and 16mc + 8 + 4hh + {0..3}.
#pragma unroll
    for (int ct = 0; ct < S::kOutTiles; ++ct) {
      const int col = 32 * ct + v_col_lane;
#pragma unroll
      for (int mc = 0; mc < 4; ++mc) {
        const int ra = 16 * mc + v_row_lane;
        const s16x4 lo = lds_read_tr(sV, v_off<D>(ra, col));
        const s16x4 hi = lds_read_tr(sV, v_off<D>(ra + 8, col));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 a = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        oacc[ct] = E::mma(a, pf[mc], oacc[ct]);
      }
    }
  }

  // ---- epilogue: one division per row, store O and the logsumexp
  float llo, lhi;
  half_pair(l_run, llo, lhi);
  const float l_tot = llo + lhi;
  if (myq < N) {
    const float inv = 1.f / l_tot;
    unsigned short* og = (unsigned short*)p.o + q_head + (long long)myq * D;
#pragma unroll
    for (int ct = 0; ct < S::kOutTiles; ++ct) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const u32x2 w = u32x2{E::pack2(oacc[ct][4 * gq + 0] * inv, oacc[ct][4 * gq + 1] * inv),
                              E::pack2(oacc[ct][4 * gq + 2] * inv, oacc[ct][4 * gq + 3] * inv)};
        *(u32x2*)(og + 32 * ct + 8 * gq + 4 * hh) = w;
      }
    }
    if (hh == 0 && p.lse != nullptr)
      p.lse[(long long)it.bh * N + myq] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

template <typename E, int D>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const FwdParams p = make_params(a, kBR);
  hipLaunchKernelGGL((fwd_mfma_kernel<E, D>), dim3(p.total_items), dim3(kThreads), 0, stream, p);
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
