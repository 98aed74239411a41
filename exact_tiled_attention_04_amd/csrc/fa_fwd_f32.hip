// Exact attention forward for float32 inputs, on the vector ALUs.
//
// Same method as the matrix-core path (tiles of K and V staged in LDS, the
// score tile kept in registers, online softmax with a running max and sum,
// one division at the end; Flash Attention page, heepie.pages.dev, "TO-BE"
// diagram and tiling section), but in fp32 arithmetic throughout, for inputs
// whose accuracy budget (1e-5 absolute on O) rules out rounding them to a
// 16-bit matrix-core type.
//
// Layout of the work: 64 query rows per workgroup of 256 threads; four
// consecutive lanes share one query row, each holding a quarter of the head
// dimension of q and of the output accumulator.  A score is the sum of the
// four lanes' partial dot products (two butterfly exchanges).  K/V tiles of
// 32 keys go through LDS; every lane of a quad reads a distinct 16-byte slice
// of a K or V row and the 16 quads of a wavefront read the same addresses
// (an LDS broadcast).
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;   // query rows per workgroup
constexpr int kKeys = 32;   // keys per K/V tile
constexpr float kLn2 = 0.69314718055994531f;

// The value of another lane of the same quad, chosen by a DPP quad_perm
// control (two bits per destination lane: the source lane within the quad).
template <int kQuadPerm>
__device__ __forceinline__ float quad_swap(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kQuadPerm, 0xf, 0xf, false));
}

template <int D>
__global__ void __launch_bounds__(kThreads) fwd_f32_kernel(FwdParams p) {
  constexpr int kVec = D / 16;  // float4 slices per lane
  constexpr int kRow4 = D / 4;  // float4 per row
  constexpr int kTile4 = kKeys * kRow4;
  static_assert(kTile4 % kThreads == 0, "tile must split evenly");
  __shared__ float4 sK[kTile4];
  __shared__ float4 sV[kTile4];

  const int tid = threadIdx.x;
  const int r = tid & 3;        // quarter of the head dimension
  const int qi = tid >> 2;      // row within the workgroup

  const WorkItem it = decode_work_item(p, blockIdx.x);
  const int N = p.N;
  const int b = it.bh / p.Hq;
  const int hq = it.bh - b * p.Hq;
  const int hk = hq / p.group;
  const long long q_head = (long long)it.bh * N * D;
  const long long kv_head = ((long long)b * p.Hkv + hk) * N * D;
  const float4* __restrict__ qg = (const float4*)((const float*)p.q + q_head);
  const float4* __restrict__ kg = (const float4*)((const float*)p.k + kv_head);
  const float4* __restrict__ vg = (const float4*)((const float*)p.v + kv_head);

  const bool causal = p.causal != 0;
  const int wl = p.window_left;
  const int q0 = it.qb * kRows;
  const int myq = q0 + qi;
  const int qlast = min(N, q0 + kRows) - 1;

  const int kend = causal ? min(N, q0 + kRows) : N;
  const int kbeg = wl >= 0 ? max(0, q0 - wl) : 0;
  const int t_beg = kbeg / kKeys;
  const int t_end = (kend + kKeys - 1) / kKeys;

  // lane r holds dims 16u + 4r .. 16u + 4r + 3 for u < kVec
  float4 qv[kVec], ov[kVec];
  const float qsgn = (float)p.q_sign;
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    qv[u] = myq < N ? qg[(long long)myq * kRow4 + 4 * u + r] : make_float4(0.f, 0.f, 0.f, 0.f);
    // the scale's sign on the query (the multiplier c below is positive)
    qv[u].x *= qsgn;
    qv[u].y *= qsgn;
    qv[u].z *= qsgn;
    qv[u].w *= qsgn;
    ov[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;

  // The next tile's K and V travel in registers while the current tile is
  // computed (one global round trip per tile is hidden behind the compute).
  constexpr int kPer = kTile4 / kThreads;  // float4 of K (and of V) per thread per tile
  float4 nk[kPer], nv[kPer];
  auto fetch = [&](int t) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + u * kThreads;
      const int key = t * kKeys + idx / kRow4;
      const int c4 = idx % kRow4;
      const bool in = t < t_end && key < N;
      nk[u] = in ? kg[(long long)key * kRow4 + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
      nv[u] = in ? vg[(long long)key * kRow4 + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  fetch(t_beg);
  for (int t = t_beg; t < t_end; ++t) {
    const int kb = t * kKeys;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      sK[tid + u * kThreads] = nk[u];
      sV[tid + u * kThreads] = nv[u];
    }
    __syncthreads();
    fetch(t + 1);
    // every key of the tile hidden from every row of the workgroup
    if ((causal && kb > qlast) || (wl >= 0 && kb + kKeys - 1 < q0 - wl)) continue;

    float s[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float part = 0.f;
#pragma unroll
      for (int u = 0; u < kVec; ++u) {
        const float4 kk = sK[j * kRow4 + 4 * u + r];
        part = __builtin_fmaf(qv[u].x, kk.x, part);
        part = __builtin_fmaf(qv[u].y, kk.y, part);
        part = __builtin_fmaf(qv[u].z, kk.z, part);
        part = __builtin_fmaf(qv[u].w, kk.w, part);
      }
      // fixed-order quad sum: ((r0 + r1) + (r2 + r3)) on every lane; the
      // partner values come through DPP quad permutations (lanes 1,0,3,2
      // and 2,3,0,1 of each quad), a vector operation each instead of an
      // LDS round trip
      const float a1 = quad_swap<0xB1>(part);
      const float p01 = (r & 1) ? (a1 + part) : (part + a1);
      const float a2 = quad_swap<0x4E>(p01);
      const float sc = (r & 2) ? (a2 + p01) : (p01 + a2);
      const int key = kb + j;
      const bool hidden = key >= N || (causal && key > myq) || (wl >= 0 && key < myq - wl);
      s[j] = hidden ? -INFINITY : sc;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      ov[u].x *= alpha;
      ov[u].y *= alpha;
      ov[u].z *= alpha;
      ov[u].w *= alpha;
    }
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c, -m_use));
      rs += pj;
#pragma unroll
      for (int u = 0; u < kVec; ++u) {
        const float4 vv = sV[j * kRow4 + 4 * u + r];
        ov[u].x = __builtin_fmaf(pj, vv.x, ov[u].x);
        ov[u].y = __builtin_fmaf(pj, vv.y, ov[u].y);
        ov[u].z = __builtin_fmaf(pj, vv.z, ov[u].z);
        ov[u].w = __builtin_fmaf(pj, vv.w, ov[u].w);
      }
    }
    l_run = l_run * alpha + rs;
  }

  if (myq < N) {
    const float inv = 1.f / l_run;
    float4* og = (float4*)((float*)p.o + q_head) + (long long)myq * kRow4;
#pragma unroll
    for (int u = 0; u < kVec; ++u)
      og[4 * u + r] = make_float4(ov[u].x * inv, ov[u].y * inv, ov[u].z * inv, ov[u].w * inv);
    if (r == 0 && p.lse != nullptr)
      p.lse[(long long)it.bh * N + myq] = (m_run + __builtin_amdgcn_logf(l_run)) * kLn2;
  }
}

template <int D>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const FwdParams p = make_params(a, kRows);
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3(p.total_items), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch<64>(a, stream) : launch<128>(a, stream);
}

long long f32_rows_per_workgroup() { return kRows; }

}  // namespace fa
