// Attention of a few query rows against a key/value cache (decoding), on
// CDNA4 (gfx950): split-KV with a logsumexp merge.
//
// The operation is the forward's (Flash Attention page, "AS-IS" diagram;
// Hacker News answers on GQA and on windows as masks), for Nq query rows that
// stand at the end of a cache of L_b keys per batch: row i sits at position
// L_b - Nq + i, so a causal mask lets it see keys j <= L_b - Nq + i.  Rows
// that see no key get o = 0, lse = -inf.
//
// Decoding reads the whole cache for very little arithmetic, so the design
// goal is HBM bandwidth, not matrix-core rate:
//
//   * one work item = one wavefront = (batch, key/value head, one or two
//     blocks of 32 query rows, split of the key range).  The rows of a work
//     item are all G * Nq query rows of the GQA group that shares the
//     key/value head, so each cached key is read once per group, not once
//     per query head; a group of four, six, ... blocks gives a wavefront
//     two blocks, whose products share each K and V read from LDS;
//   * the visible key range of a (batch, head) is cut into equal splits so
//     that the grid holds enough wavefronts to keep HBM busy even for one
//     sequence; each split writes its normalised partial output and its
//     logsumexp, and a second kernel merges the splits:
//         lse = log sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) o_s
//     (the identity the Flash Attention page's tiling section and the
//     FlashAttention quiz, question 4, rest on: blocks rescaled by their
//     normalisation factors sum to the exact result).  With one split the
//     kernel writes o and lse directly;
//   * every wavefront streams its own 32-key K and V tiles into its own LDS
//     region with direct-to-LDS buffer loads, kStages tiles deep, so no
//     workgroup barrier is ever needed; keys past the batch's length lie
//     outside the buffer's range and arrive as zeros (never NaN);
//   * the per-tile arithmetic is the forward's: S^T = K Q^T and
//     O^T += V^T P^T on v_mfma_f32_32x32x16_{bf16,f16}, an online softmax with
//     a lazily moved reference max, V through the transposing LDS read.
//
// Two cache layouts share the kernel: a contiguous cache [B][Hkv][Nk][d]
// with per-batch lengths, and a paged cache [pages][page_size][Hkv][d] with a
// per-batch table of page indices (page_size a multiple of 32, so a tile never
// straddles two pages, or 16, when each half of a tile comes from its own
// page).  Page indices outside [0, pages) read as zeros.
#include "fa_internal.h"
#include "fa_decode.h"
#include "fa_mfma_common.h"

#include <climits>
#include <mutex>

namespace fa {
namespace {

using namespace mfma;

constexpr int kTile = 32;  // keys per tile
// One wavefront per workgroup with two 16 KiB stages (d = 128) lets five
// wavefronts share a compute unit's LDS, which kept the most bytes in flight
// among the shapes measured (1-4 waves per workgroup, 2-4 stages).
#ifndef FA_DEC_WAVES
#define FA_DEC_WAVES 1
#endif
#ifndef FA_DEC_STAGES
#define FA_DEC_STAGES 2
#endif
constexpr int kWaves = FA_DEC_WAVES;    // independent wavefronts per workgroup
constexpr int kStages = FA_DEC_STAGES;  // K/V tiles in LDS per wavefront
// A GQA group with an even number (at least four) of 32-row blocks gives each
// wavefront two of them, so that every K and V tile it copies into LDS and
// reads from there serves 64 rows (decode_row_blocks_per_item).
#ifndef FA_DEC_MAX_RB
#define FA_DEC_MAX_RB 2
#endif
constexpr int kMaxRowBlocks = FA_DEC_MAX_RB;
static_assert(kStages >= 2 && kStages <= 4, "stages");
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleSlack = 8.0f;   // as in the forward: probabilities stay <= 2^8

template <int D>
struct DShape {
  static constexpr int kSteps = D / 16;     // MFMA k-steps of the score product
  static constexpr int kOutTiles = D / 32;  // 32-wide output channel tiles
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;     // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;
  static constexpr int kLoads = kTile / kRowsPerLoad;  // 1-KiB loads per tensor per tile
  static constexpr int kTileElems = kTile * D;
};

// LDS tile layouts (row-major [key][dim], 16-byte chunks XOR-permuted by a
// function of the row), conflict-free for the two read patterns of a tile:
// 16-byte reads of K by 32 lanes on 32 consecutive rows, and the transposing
// read of V by 16-lane groups on 4 consecutive rows x 32 bytes.
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

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x = min(x, __shfl_xor(x, m, kWaveSize));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x = max(x, __shfl_xor(x, m, kWaveSize));
  return x;
}

template <int kOutstanding>
__device__ __forceinline__ void wait_loads() {
  static_assert(kOutstanding >= 0 && kOutstanding < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kOutstanding) : "memory");
}

// A kernel-uniform int read through the scalar cache (constant address
// space): it counts against lgkmcnt, not vmcnt, so reading a page index never
// waits for the tile copies in flight.
typedef __attribute__((address_space(4))) const int const_int_t;
__device__ __forceinline__ int scalar_load(const int* ptr, long long idx) {
  return ((const_int_t*)ptr)[idx];
}

// Where one tile of one tensor comes from: a buffer resource and the byte
// offset of the tile's first row within it.
struct TileSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  int soff;
};

template <typename E, int D, bool kPaged>
struct Decode {
  using S = DShape<D>;

  // The buffer and offset of tile t (keys 32t .. 32t+31) of this (batch,
  // key/value head) in K (or V).
  static __device__ __forceinline__ TileSrc tile_src(const DecodeParams& p, const void* base, int b, int hk,
                                                     int L, int t) {
    TileSrc r;
    const int row_bytes = p.row_stride * 2;
    if constexpr (kPaged) {
      // wave-uniform by construction; readfirstlane keeps the integer
      // division's result in scalar registers, so the table read below is a
      // scalar load
      const int key0 = t * kTile;
      const int page_slot = __builtin_amdgcn_readfirstlane(key0 / p.page_size);
      const int in_page = key0 - page_slot * p.page_size;
      const int page = scalar_load(p.block_table, (long long)b * p.max_pages + page_slot);
      const bool ok = page >= 0 && page < p.num_pages;
      // rows of this page that belong to the sequence: the rest read as zeros
      const int rows = min(p.page_size, L - page_slot * p.page_size);
      const char* pb = (const char*)base + ((long long)(ok ? page : 0) * p.page_size * p.row_stride + (long long)hk * D) * 2;
      const int bytes = ok && rows > 0 ? (rows - 1) * row_bytes + S::kRowBytes : 0;
      r.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)pb, 0, bytes, kBufferFlags);
      r.soff = in_page * row_bytes;
    } else {
      const char* hb = (const char*)base + ((long long)b * p.batch_stride + (long long)hk * p.head_stride) * 2;
      const int bytes = L > 0 ? (L - 1) * row_bytes + S::kRowBytes : 0;
      r.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)hb, 0, bytes, kBufferFlags);
      r.soff = t * kTile * row_bytes;
    }
    return r;
  }

  // 16-token pages: the buffer of the page holding keys 16 slot ..
  // 16 slot + 15 (slot = 2t + half), based 16 half rows before the page so
  // that the tile's row offsets (rows 16 half .. 16 half + 15) address it,
  // and bounded to the sequence's rows of the page (offsets below 16 half
  // rows are never used).
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t half_src(const DecodeParams& p, const void* base,
                                                                   int b, int hk, int L, int slot, int half) {
    const int row_bytes = p.row_stride * 2;
    // the entry is read unconditionally (clamped into the table's row), so
    // the lookups of both halves issue together; a slot past the sequence
    // (slot * 16 >= L; below that slot < max_pages, as L <= 16 max_pages)
    // ignores what it read
    const bool live = slot * 16 < L;
    const int entry = scalar_load(p.block_table, (long long)b * p.max_pages + min(slot, p.max_pages - 1));
    const int page = live ? entry : -1;
    const bool ok = page >= 0 && page < p.num_pages;
    const int rows = min(16, L - slot * 16);
    const char* pb = (const char*)base + ((long long)(ok ? page : 0) * 16 * p.row_stride + (long long)hk * D) * 2 -
                     (long long)half * 16 * row_bytes;
    const int bytes = ok && rows > 0 ? half * 16 * row_bytes + (rows - 1) * row_bytes + S::kRowBytes : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)pb, 0, bytes, kBufferFlags);
  }

  // Start copying tile t of K and V into LDS (2 * kLoads loads per lane).
  static __device__ __forceinline__ void issue(const DecodeParams& p, int b, int hk, int L, int t,
                                               const int* ok_, const int* ov_, unsigned short* kdst,
                                               unsigned short* vdst) {
    if constexpr (kPaged) {
      if (p.page_size < kTile) {
        // load u covers rows u * kRowsPerLoad ..: the first kLoads / 2 loads
        // are the tile's first 16 rows
        static_assert(S::kLoads % 2 == 0 && S::kRowsPerLoad <= 16, "a load must stay within one half tile");
        __amdgpu_buffer_rsrc_t kr[2], vr[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          kr[h] = half_src(p, p.k, b, hk, L, 2 * t + h, h);
          vr[h] = half_src(p, p.v, b, hk, L, 2 * t + h, h);
        }
#pragma unroll
        for (int u = 0; u < S::kLoads; ++u) {
          const int o = ok_[u];
          __builtin_amdgcn_raw_ptr_buffer_load_lds(kr[u >= S::kLoads / 2], (lds_void_t*)(kdst + u * 512), 16, o, 0,
                                                   0, 0);
        }
#pragma unroll
        for (int u = 0; u < S::kLoads; ++u) {
          const int o = ov_[u];
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vr[u >= S::kLoads / 2], (lds_void_t*)(vdst + u * 512), 16, o, 0,
                                                   0, 0);
        }
        return;
      }
    }
    const TileSrc ks = tile_src(p, p.k, b, hk, L, t);
    const TileSrc vs = tile_src(p, p.v, b, hk, L, t);
#pragma unroll
    for (int u = 0; u < S::kLoads; ++u) {
      const int o = ok_[u], so = ks.soff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ks.rsrc, (lds_void_t*)(kdst + u * 512), 16, o, so, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < S::kLoads; ++u) {
      const int o = ov_[u], so = vs.soff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vs.rsrc, (lds_void_t*)(vdst + u * 512), 16, o, so, 0, 0);
    }
  }
};

template <typename E, int D, bool kPaged, int kRB>
__global__ void __launch_bounds__(kWaves * kWaveSize) decode_split_kernel(DecodeParams p) {
  using S = DShape<D>;
  using K = Decode<E, D, kPaged>;
  __shared__ __attribute__((aligned(16))) unsigned short smem[kWaves][kStages][2][S::kTileElems];

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  // Workgroups go to the 8 XCDs round-robin (workgroup id mod 8).  A unit
  // (batch * Hkv + head, split) goes to XCD unit mod 8 with its row items
  // together (they stream the same tiles, shared through that XCD's L2), so
  // every XCD gets units of every sequence: caches of different lengths do
  // not leave some XCDs with far more work than others.  The grid holds
  // 8 * ceil(units / 8) units; the missing ones return at once.
  int item;
  if constexpr (kWaves == 1) {
    const int xcd = blockIdx.x % 8;
    const int r = blockIdx.x / 8;
    const int u_local = r / p.n_row_items;
    const int unit = 8 * u_local + xcd;
    if (unit >= p.total_items / p.n_row_items) return;
    item = unit * p.n_row_items + (r - u_local * p.n_row_items);
  } else {
    item = xcd_slice_index(blockIdx.x, gridDim.x) * kWaves + wave;
    if (item >= p.total_items) return;  // whole wavefronts only; no barrier follows
  }

  const int ri = item % p.n_row_items;
  const int rest = item / p.n_row_items;
  const int s = rest % p.n_splits;
  const int bk = rest / p.n_splits;
  const int b = bk / p.Hkv;
  const int hk = bk - b * p.Hkv;
  const int L = min(max(p.seqlens ? scalar_load(p.seqlens, b) : p.Nk, 0), p.Nk);

  const int l32 = lane & 31, hh = lane >> 5;
  // the wavefront's kRB blocks of 32 rows (rows of the group's G * Nq);
  // lane l32 holds row l32 of each
  bool valid[kRB], any[kRB];
  int lo[kRB];
  unsigned span[kRB];
  long long out_row[kRB];
  int wlo = INT_MAX, whi = -1;
  // keys every valid row of block j sees: [clean_lo[j], clean_hi[j]] (empty
  // when some valid row sees no key); a tile inside it needs no mask
  int clean_lo[kRB], clean_hi[kRB];
#pragma unroll
  for (int j = 0; j < kRB; ++j) {
    const int r = (ri * kRB + j) * 32 + l32;
    valid[j] = r < p.group * p.Nq;
    const int g = valid[j] ? r / p.Nq : 0;
    const int i = valid[j] ? r - g * p.Nq : 0;
    const int pos = L - p.Nq + i;
    lo[j] = p.window_left >= 0 ? max(0, pos - p.window_left) : 0;
    const int hi = p.causal ? min(pos, L - 1) : L - 1;
    any[j] = valid[j] && hi >= lo[j];
    span[j] = (unsigned)(hi - lo[j]);
    out_row[j] = ((long long)b * p.Hq + hk * p.group + g) * p.Nq + i;
    if (any[j]) {
      wlo = min(wlo, lo[j]);
      whi = max(whi, hi);
    }
    clean_lo[j] = __builtin_amdgcn_readfirstlane(wave_max(valid[j] ? (any[j] ? lo[j] : INT_MAX) : INT_MIN));
    clean_hi[j] = __builtin_amdgcn_readfirstlane(wave_min(valid[j] ? (any[j] ? hi : INT_MIN) : INT_MAX));
  }

  // this split's tiles: the s-th chunk of tiles_per_split tiles of the range
  // the wavefront's rows need (a chunk size fixed on the host from the
  // cache capacity, so short sequences leave their last splits empty and no
  // split of a long one is longer than any other)
  // (the reductions leave the same value in every lane; readfirstlane makes
  // that known to the compiler, so the tile loop and every copy's buffer
  // resource and offset stay in scalar registers instead of being wrapped in
  // a loop over the distinct values of the lanes)
  wlo = __builtin_amdgcn_readfirstlane(wave_min(wlo));
  whi = __builtin_amdgcn_readfirstlane(wave_max(whi));
  int t_beg = 0, t_end = 0;
  if (whi >= wlo) {
    const int tb0 = wlo / kTile, tb1 = whi / kTile + 1;
    const int per = max(p.tiles_per_split, (tb1 - tb0 + p.n_splits - 1) / p.n_splits);
    t_beg = min(tb1, tb0 + s * per);
    t_end = min(tb1, t_beg + per);
  }

  f32x16 oacc[kRB][S::kOutTiles];
#pragma unroll
  for (int j = 0; j < kRB; ++j)
#pragma unroll
    for (int ct = 0; ct < S::kOutTiles; ++ct) oacc[j][ct] = f32x16{};
  float m_use[kRB], l_run[kRB];
#pragma unroll
  for (int j = 0; j < kRB; ++j) {
    m_use[j] = -INFINITY;
    l_run[j] = 0.f;
  }

  if (t_beg < t_end) {
    // query rows as the B operand
    u32x4 qf[kRB][S::kSteps];
#pragma unroll
    for (int j = 0; j < kRB; ++j) {
      const unsigned short* qrow = (const unsigned short*)p.q + out_row[j] * D;
#pragma unroll
      for (int kc = 0; kc < S::kSteps; ++kc)
        qf[j][kc] = valid[j] ? q_signed16(*(const u32x4*)(qrow + 16 * kc + 8 * hh), p.q_sign) : u32x4{0u, 0u, 0u, 0u};
    }

    // per-lane copy offsets: lane fills LDS bytes 16 lane .. +15 of each 1-KiB
    // piece u, i.e. row u * kRowsPerLoad + lane / kChunks, physical chunk
    // lane % kChunks, so it fetches the logical chunk the swizzle maps there
    int ok_[S::kLoads], ov_[S::kLoads];
    const int row_bytes = p.row_stride * 2;
#pragma unroll
    for (int u = 0; u < S::kLoads; ++u) {
      const int row = u * S::kRowsPerLoad + lane / S::kChunks;
      const int pch = lane % S::kChunks;
      ok_[u] = row * row_bytes + ((pch ^ k_swz<D>(row)) << 4);
      ov_[u] = row * row_bytes + ((pch ^ v_swz<D>(row)) << 4);
    }
    const int g16 = lane >> 4, gi = lane & 15;
    const int v_row_lane = 4 * hh + (gi >> 2);
    const int v_col_lane = 16 * (g16 & 1) + 4 * (gi & 3);
    const float c = p.scale_log2;
    unsigned short* my = &smem[wave][0][0][0];

    // prologue: the first kStages - 1 tiles
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j)
      if (t_beg + j < t_end) K::issue(p, b, hk, L, t_beg + j, ok_, ov_, my + (2 * j) * S::kTileElems,
                                      my + (2 * j + 1) * S::kTileElems);

    for (int t = t_beg; t < t_end; ++t) {
      const int jt = t - t_beg;
      const int st = jt % kStages;
      const unsigned short* kC = my + (2 * st) * S::kTileElems;
      const unsigned short* vC = my + (2 * st + 1) * S::kTileElems;
      // refill the stage read in the previous step (its reads are done)
      if (t + kStages - 1 < t_end) {
        const int sn = (jt + kStages - 1) % kStages;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        K::issue(p, b, hk, L, t + kStages - 1, ok_, ov_, my + (2 * sn) * S::kTileElems,
                 my + (2 * sn + 1) * S::kTileElems);
        wait_loads<(kStages - 1) * 2 * S::kLoads>();  // tile t has landed
      } else {
        wait_loads<0>();
      }

      // scores S^T = K Q^T for keys 32t .. 32t+31; each K read serves every
      // row block
      f32x16 sacc[kRB];
#pragma unroll
      for (int j = 0; j < kRB; ++j) sacc[j] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < S::kSteps; ++kc) {
        const u32x4 a = *(const u32x4*)(kC + k_off<D>(l32, 2 * kc + hh));
#pragma unroll
        for (int j = 0; j < kRB; ++j) sacc[j] = E::mma(a, qf[j][kc], sacc[j]);
      }
      u32x4 pf[kRB][2];
#pragma unroll
      for (int j = 0; j < kRB; ++j) {
        // mask: key kb + 8(e/4) + 4hh + e%4 is visible iff lo <= key <= hi;
        // tiles every valid row sees whole skip it (rows past the group's
        // are never stored)
        if (t * kTile < clean_lo[j] || t * kTile + kTile - 1 > clean_hi[j]) {
          const int base = t * kTile + 4 * hh - lo[j];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int off = 8 * (e >> 2) + (e & 3);
            sacc[j][e] = (any[j] && (unsigned)(base + off) <= span[j]) ? sacc[j][e] : -INFINITY;
          }
        }
        // online softmax (base 2, scale folded into the exponent)
        float mx = sacc[j][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sacc[j][e]);
        float mlo, mhi;
        half_pair(mx, mlo, mhi);
        mx = fmaxf(mlo, mhi) * c;
        const bool bump = mx > m_use[j] + kRescaleSlack;
        const float alpha = bump ? __builtin_amdgcn_exp2f(m_use[j] - mx) : 1.f;
        m_use[j] = bump ? mx : m_use[j];
        const float m_exp = (m_use[j] == -INFINITY) ? 0.f : m_use[j];
        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sacc[j][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][e], c, -m_exp));
          part[e & 3] += sacc[j][e];
        }
        l_run[j] = __builtin_fmaf(l_run[j], alpha, (part[0] + part[1]) + (part[2] + part[3]));
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
          for (int ct = 0; ct < S::kOutTiles; ++ct) oacc[j][ct] *= alpha;
        }
#pragma unroll
        for (int mc = 0; mc < 2; ++mc)
          pf[j][mc] = u32x4{E::pack2(sacc[j][8 * mc + 0], sacc[j][8 * mc + 1]),
                            E::pack2(sacc[j][8 * mc + 2], sacc[j][8 * mc + 3]),
                            E::pack2(sacc[j][8 * mc + 4], sacc[j][8 * mc + 5]),
                            E::pack2(sacc[j][8 * mc + 6], sacc[j][8 * mc + 7])};
      }
      // O^T += V^T P^T; k-step mc covers keys 16mc .. 16mc+15 in the
      // accumulator's order (half-wave hh holds 16mc + 4hh + {0..3} and
      // 16mc + 8 + 4hh + {0..3}); each V read serves every row block
#pragma unroll
      for (int ct = 0; ct < S::kOutTiles; ++ct) {
        const int col = 32 * ct + v_col_lane;
#pragma unroll
        for (int mc = 0; mc < 2; ++mc) {
          const int ra = 16 * mc + v_row_lane;
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lds_read_tr(vC, v_off<D>(ra, col)));
          const u32x2 hi2 = __builtin_bit_cast(u32x2, lds_read_tr(vC, v_off<D>(ra + 8, col)));
          const u32x4 vt = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
#pragma unroll
          for (int j = 0; j < kRB; ++j) oacc[j][ct] = E::mma(vt, pf[j][mc], oacc[j][ct]);
        }
      }
    }
  }

  // epilogue: this split's normalised output and logsumexp (o = 0 and
  // lse = -inf where the row saw no key)
#pragma unroll
  for (int j = 0; j < kRB; ++j) {
    float llo, lhi;
    half_pair(l_run[j], llo, lhi);
    const float l_tot = llo + lhi;
    if (!valid[j]) continue;
    const bool seen = l_tot > 0.f;
    const float inv = seen ? 1.f / l_tot : 0.f;
    const float lse = seen ? (m_use[j] + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    if (p.n_splits == 1) {
      unsigned short* og = (unsigned short*)p.o + out_row[j] * D;
#pragma unroll
      for (int ct = 0; ct < S::kOutTiles; ++ct) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const u32x2 w = u32x2{E::pack2(oacc[j][ct][4 * gq + 0] * inv, oacc[j][ct][4 * gq + 1] * inv),
                                E::pack2(oacc[j][ct][4 * gq + 2] * inv, oacc[j][ct][4 * gq + 3] * inv)};
          *(u32x2*)(og + 32 * ct + 8 * gq + 4 * hh) = w;
        }
      }
      if (hh == 0 && p.lse != nullptr) p.lse[out_row[j]] = lse;
    } else {
      const long long prow = (long long)s * p.rows + out_row[j];
      float* po = p.part_o + prow * D;
#pragma unroll
      for (int ct = 0; ct < S::kOutTiles; ++ct) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const float4 w = make_float4(oacc[j][ct][4 * gq + 0] * inv, oacc[j][ct][4 * gq + 1] * inv,
                                       oacc[j][ct][4 * gq + 2] * inv, oacc[j][ct][4 * gq + 3] * inv);
          *(float4*)(po + 32 * ct + 8 * gq + 4 * hh) = w;
        }
      }
      if (hh == 0) p.part_lse[prow] = lse;
    }
  }
}

// Merge of the splits: one wavefront per output row.  Lane j holds the
// logsumexp of splits j and j + 64; the row max and the weights come from
// wavefront reductions, then every lane accumulates its D/64 channels over the
// splits in order (deterministic), eight loads in flight at a time.
constexpr int kMergeRows = 4;  // rows (wavefronts) per workgroup

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, kWaveSize));
  return x;
}

template <typename E, int D>
__global__ void __launch_bounds__(kMergeRows * kWaveSize) decode_merge_kernel(DecodeParams p) {
  constexpr int kPer = D / kWaveSize;  // channels per lane (1 or 2)
  const int lane = threadIdx.x & (kWaveSize - 1);
  const long long row = (long long)blockIdx.x * kMergeRows + threadIdx.x / kWaveSize;
  if (row >= p.rows) return;
  const int S = p.n_splits;  // <= 128
  const float l0 = lane < S ? p.part_lse[(long long)lane * p.rows + row] : -INFINITY;
  const float l1 = lane + kWaveSize < S ? p.part_lse[(long long)(lane + kWaveSize) * p.rows + row] : -INFINITY;
  const float mx = wave_max_f(fmaxf(l0, l1));
  // weights exp(lse_s - max): 0 for empty splits, and everything 0 when the
  // row saw no key anywhere
  const float w0 = mx == -INFINITY ? 0.f : __expf(l0 - mx);
  const float w1 = mx == -INFINITY ? 0.f : __expf(l1 - mx);
  float acc[kPer];
#pragma unroll
  for (int c = 0; c < kPer; ++c) acc[c] = 0.f;
  float l = 0.f;
  const float* po = p.part_o + row * D + kPer * lane;
  const long long sstride = p.rows * D;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8][kPer];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int c = 0; c < kPer; ++c) v[u][c] = s0 + u < S ? po[(s0 + u) * sstride + c] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sj = s0 + u;
      const float w = __shfl(sj < kWaveSize ? w0 : w1, sj & (kWaveSize - 1), kWaveSize);
      if (sj < S) {
        l += w;
#pragma unroll
        for (int c = 0; c < kPer; ++c) acc[c] = __builtin_fmaf(w, v[u][c], acc[c]);
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  unsigned short* og = (unsigned short*)p.o + row * D + kPer * lane;
  if constexpr (kPer == 2) {
    *(unsigned*)og = E::pack2(acc[0] * inv, acc[1] * inv);
  } else {
    og[0] = (unsigned short)(E::pack2(acc[0] * inv, 0.f) & 0xffffu);
  }
  if (lane == 0 && p.lse != nullptr) p.lse[row] = l > 0.f ? mx + __logf(l) : -INFINITY;
}

template <typename E, int D, int kRB>
void launch_split(const DecodeParams& p, int blocks, hipStream_t stream) {
  if (p.block_table)
    hipLaunchKernelGGL((decode_split_kernel<E, D, true, kRB>), dim3(blocks), dim3(kWaves * kWaveSize), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<E, D, false, kRB>), dim3(blocks), dim3(kWaves * kWaveSize), 0, stream,
                       p);
}

template <typename E, int D>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int units = p.total_items / p.n_row_items;
  const int blocks = kWaves == 1 ? 8 * ((units + 7) / 8) * p.n_row_items : (p.total_items + kWaves - 1) / kWaves;
  if (p.rb_per_item == 2)
    launch_split<E, D, 2>(p, blocks, stream);
  else
    launch_split<E, D, 1>(p, blocks, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  const long long mblocks = (p.rows + kMergeRows - 1) / kMergeRows;
  hipLaunchKernelGGL((decode_merge_kernel<E, D>), dim3((unsigned)mblocks), dim3(kMergeRows * kWaveSize), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d, bool f16, hipStream_t stream) {
  if (f16) return d == 64 ? launch_t<F16, 64>(p, stream) : launch_t<F16, 128>(p, stream);
  return d == 64 ? launch_t<Bf16, 64>(p, stream) : launch_t<Bf16, 128>(p, stream);
}

int decode_waves_per_workgroup() { return kWaves; }

// Two blocks per wavefront only for an even count of at least four: on
// MI355X (16k-token caches, GQA 4:1, each count at the split count its own
// rule picks) one block per wavefront was 5-12% faster for 2, 3 and 5 blocks
// (more wavefronts, fewer registers each, no half-empty wavefront) and two
// were 1-7% faster for 4 and 8 (each K/V tile copied into LDS once for 64
// rows instead of 32).
int decode_row_blocks_per_item(int n_row_blocks) {
  return n_row_blocks >= 4 && n_row_blocks % 2 == 0 && kMaxRowBlocks >= 2 ? 2 : 1;
}

// Scratch of the allocation-free decoding entry point: the splits' partial
// outputs and logsumexps live in this file-scope device array instead of a
// caller's workspace.  Each GPU the library runs on holds its own copy at its
// own address until the process ends.  In host code the array's name is a
// host-side stand-in, never a device address: the address every launch uses
// comes from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

size_t decode_scratch_bytes() { return kDecodeScratchBytes; }

hipError_t decode_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(a);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace fa
