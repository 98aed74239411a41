// Internal declarations shared by the C-ABI wrapper and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {

// Validated arguments of one forward call (sizes already checked on the host).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null: skip writing the logsumexp
  int B, Hq, Hkv, N, d;
  int causal;
  int window_left;  // -1 = no window
  float scale;      // any finite value
  // packed sequences of different lengths (null: one N for all): q [total_q]
  // [Hq][d], k, v [total_k][Hkv][d], sequence b owning rows cu_q[b] ..
  // cu_q[b+1]-1 and keys cu_k[b] .. cu_k[b+1]-1; N is then the longest query
  // count and max_k the longest key count
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0, max_k = 0;
};

// Kernel-side copy of the arguments plus derived constants.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N;
  int group;         // Hq / Hkv: query heads per key/value head
  int causal;
  int window_left;
  int n_qblocks;     // ceil(N / rows per workgroup)
  int total_items;   // B * Hq * n_qblocks
  float scale_log2;  // |scale| * log2(e) (1 * log2(e) for a zero scale): scores
                     // go straight into exp2 (FP8: times the Q and K scales)
  int q_sign;        // sign of the scale: +1; -1 (queries negated in registers,
                     // so the positive multiplier above gives the same scores);
                     // 0 (queries read as zeros: every visible score is 0)
  float o_mult;      // multiplier on the output: the V scale of FP8 inputs, else 1
  const int* cu_q;   // packed variable-length sequences (null: fixed N), as FwdArgs
  const int* cu_k;
  int total_q, total_k, max_k;
};

// Workgroup -> (batch*head, query block) mapping.
//
// Workgroups are handed to the 8 XCDs of the chip round-robin (workgroup id
// modulo 8), and each XCD has its own L2.  The mapping gives every XCD a
// contiguous slice of a logical order in which the query blocks of the query
// heads that share one key/value head are adjacent, so the K/V tiles that
// those workgroups stream are shared through one L2.  With a causal mask the
// logical order within a head group runs from the last query block (the most
// key tiles) to the first, so long workgroups start early.
struct WorkItem {
  int bh;  // b * Hq + query head
  int qb;  // query block index
};

// Position of workgroup `id` in the logical order: the 8 XCDs take
// contiguous slices of it.
__device__ __forceinline__ int xcd_slice_index(int id, int total_items) {
  constexpr int NXCD = 8;
  const int xcd = id % NXCD;
  const int r = id / NXCD;
  const int per = total_items / NXCD;
  const int rem = total_items % NXCD;
  return xcd * per + (xcd < rem ? xcd : rem) + r;
}

__device__ __forceinline__ WorkItem decode_work_item(const FwdParams& p, int id) {
  const int L = xcd_slice_index(id, p.total_items);
  const int per_group = p.group * p.n_qblocks;
  const int gidx = L / per_group;
  const int w = L - gidx * per_group;
  const int qrank = w / p.group;
  const int hg = w - qrank * p.group;
  const int b = gidx / p.Hkv;
  const int hk = gidx - b * p.Hkv;
  WorkItem it;
  it.bh = b * p.Hq + hk * p.group + hg;
  it.qb = p.causal ? (p.n_qblocks - 1 - qrank) : qrank;
  return it;
}

// The kernels take each row's maximum over the raw products q.k and multiply
// by the scale afterwards, which is only right for a positive multiplier.
// scale * q.k equals |scale| * (-q).k for a negative scale (negating a query
// flips sign bits: exact), and 0 * q.k equals any positive multiple of 0.k,
// so the kernels get a positive multiplier and the sign to apply to Q.
template <typename P>
inline void set_score_scale(P& p, float scale) {
  p.q_sign = scale > 0.f ? 1 : (scale < 0.f ? -1 : 0);
  p.scale_log2 = (scale != 0.f ? __builtin_fabsf(scale) : 1.f) * 1.4426950408889634f;
}

inline FwdParams make_params(const FwdArgs& a, int rows_per_wg) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.N = a.N;
  p.group = a.Hq / a.Hkv;
  p.causal = a.causal ? 1 : 0;
  // a window of N-1 or more keys reaches back past key 0 and hides nothing
  // (packed sequences: of the longest key count - 1 or more)
  const int span = a.cu_q ? (a.N > a.max_k ? a.N : a.max_k) : a.N;
  p.window_left = (a.window_left >= span - 1) ? -1 : a.window_left;
  p.n_qblocks = (a.N + rows_per_wg - 1) / rows_per_wg;
  p.total_items = a.B * a.Hq * p.n_qblocks;
  set_score_scale(p, a.scale);
  p.o_mult = 1.f;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.max_k = a.max_k;
  return p;
}

// Validated arguments of one backward call.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* work;  // 2 * B * Hq * N floats (packed: 2 * Hq * total_q): row terms D_i, then lse_i * log2(e)
  int B, Hq, Hkv, N, d;  // packed sequences: N = max_seqlen_q
  int causal;
  int window_left;
  float scale;
  // packed variable-length sequences (null: fixed N), as FwdArgs: q, o, dout,
  // dq [total_q][Hq][d], k, v, dk, dv [total_k][Hkv][d], lse [Hq][total_q]
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0, max_k = 0;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [B][Hq][N] (packed: [Hq][total_q]): -sum_c dout * o
  float* lse2;   // same layout: lse * log2(e), +inf where lse = -inf
  long long rows;  // B * Hq * N (packed: Hq * total_q)
  int B, Hq, Hkv, N;  // packed: N = max_seqlen_q
  int group;
  int causal;
  int window_left;   // -1 = none (normalised: a window reaching key 0 from every row becomes -1)
  int n_blocks;      // ceil(N / 128): query blocks (dQ)
  int n_kblocks;     // key blocks of the dK/dV launch (its block size: bwd_keys_per_workgroup)
  int items_dq;      // B * Hq * n_blocks
  int items_dkv;     // B * Hkv * n_kblocks
  float scale;
  float scale_log2;
  const int* cu_q;   // packed sequences, as BwdArgs (null: fixed N)
  const int* cu_k;
  int total_q, total_k, max_k;
};

inline BwdParams make_bwd_params(const BwdArgs& a, int rows_per_wg) {
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.dout = a.dout;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  const bool packed = a.cu_q != nullptr;
  p.rows = packed ? (long long)a.Hq * a.total_q : (long long)a.B * a.Hq * a.N;
  p.delta = a.work;
  p.lse2 = a.work + p.rows;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.N = a.N;
  p.group = a.Hq / a.Hkv;
  p.causal = a.causal ? 1 : 0;
  // a row at key position pos sees keys from pos - window_left on: with
  // positions below the key count, a window of that many keys or more
  // reaches key 0 from every row
  const int nk = packed ? a.max_k : a.N;
  p.window_left = (a.window_left >= nk - 1) ? -1 : a.window_left;
  p.n_blocks = (a.N + rows_per_wg - 1) / rows_per_wg;
  p.n_kblocks = (nk + rows_per_wg - 1) / rows_per_wg;
  p.items_dq = a.B * a.Hq * p.n_blocks;
  p.items_dkv = a.B * a.Hkv * p.n_kblocks;
  p.scale = a.scale;
  // any sign: the backward masks after the exponent, and rebuilds P from the
  // scaled score and the saved logsumexp (no row maximum is taken)
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.max_k = a.max_k;
  return p;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_f16(const BwdArgs& a, hipStream_t stream);
long long bwd_rows_per_workgroup();            // query rows of a dQ workgroup
long long bwd_keys_per_workgroup(int d);       // keys of a dK/dV workgroup at head dimension d

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
// q, k, v hold E4M3 bytes standing for byte * scale; o is bfloat16.
hipError_t launch_fwd_fp8(const FwdArgs& a, float q_scale, float k_scale, float v_scale, hipStream_t stream);

// Query rows handled by one workgroup of each kernel.
long long mfma_rows_per_workgroup();
long long f32_rows_per_workgroup();
long long fp8_rows_per_workgroup();

// Largest B*Hq*n_qblocks a single launch accepts (grid.x limit).
constexpr long long kMaxGridItems = 2147483647LL;

}  // namespace fa
