// C-ABI entry points: argument validation on the host, then the kernel launches.
// The operation, layouts, ownership and error behaviour are specified in
// include/fa.h.
#include "fa.h"

#include <algorithm>
#include <vector>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa_internal.h"
#include "fa_decode.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

size_t elem_size(int dt) { return dt == FA_DTYPE_F32 ? 4 : 2; }

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Checks shared by the forward and the backward.  Returns FA_OK with
// *empty = true when there is nothing to compute.
int check_sizes(int B, int Hq, int Hkv, int N, int d, int window_left, float scale, int dtype,
                bool* empty) {
  *empty = false;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_UNSUPPORTED, "unknown dtype %d", static_cast<int>(dtype));
  if (B < 0 || Hq < 0 || Hkv < 0 || N < 0 || d < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size (B=%d Hq=%d Hkv=%d N=%d d=%d)", B, Hq, Hkv, N, d);
  if (B == 0 || Hq == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  if (Hkv == 0 || Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
  if (window_left < -1)
    return fail(FA_ERR_INVALID_ARG, "window_left=%d (must be -1 or >= 0)", window_left);
  if (!std::isfinite(scale))
    return fail(FA_ERR_INVALID_ARG, "scale is not finite");
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128)", d);
  return FA_OK;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
        int N, int d, int causal, int window_left, float scale, void* stream, int dtype) {
  g_last_error[0] = '\0';
  bool empty;
  if (int st = check_sizes(B, Hq, Hkv, N, d, window_left, scale, dtype, &empty)) return st;
  if (empty) return FA_OK;  // nothing to compute
  if (!q || !k || !v || !o)
    return fail(FA_ERR_INVALID_ARG, "null q/k/v/o pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_MISALIGNED, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4))
    return fail(FA_ERR_MISALIGNED, "lse must be 4-byte aligned");
  // o and lse must not overlap each other (inputs are checked loosely: exact
  // extents of device allocations are unknown here, so only the spans implied
  // by the sizes are compared).
  const uint64_t n_o = (uint64_t)B * Hq * N * d * elem_size(dtype);
  const uint64_t n_kv = (uint64_t)B * Hkv * N * d * elem_size(dtype);
  if (overlap(o, n_o, q, n_o) || overlap(o, n_o, k, n_kv) || overlap(o, n_o, v, n_kv))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (lse) {
    const uint64_t n_l = (uint64_t)B * Hq * N * sizeof(float);
    if (overlap(lse, n_l, o, n_o) || overlap(lse, n_l, q, n_o) || overlap(lse, n_l, k, n_kv) ||
        overlap(lse, n_l, v, n_kv))
      return fail(FA_ERR_INVALID_ARG, "lse overlaps o or an input");
  }
  // K/V tiles are addressed with 32-bit byte offsets within one head
  // (a few tiles of slack past the end)
  if ((uint64_t)N * d * elem_size(dtype) + (1u << 20) > (uint64_t)INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "N=%d too long for d=%d (one head must stay below 2 GiB)", N, d);
  const long long rows = dtype == FA_DTYPE_F32 ? fa::f32_rows_per_workgroup() : fa::mfma_rows_per_workgroup();
  const long long items = (long long)B * Hq * ((N + rows - 1) / rows);
  if (items > fa::kMaxGridItems)
    return fail(FA_ERR_UNSUPPORTED, "B*Hq*ceil(N/%lld)=%lld exceeds one launch", rows, items);

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.causal = causal;
  a.window_left = window_left;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (dtype) {
    case FA_DTYPE_BF16: e = fa::launch_fwd_bf16(a, s); break;
    case FA_DTYPE_F16: e = fa::launch_fwd_f16(a, s); break;
    default: e = fa::launch_fwd_f32(a, s); break;
  }
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return FA_OK;
}

int run_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_q, const int* cu_k,
               int B, int Hq, int Hkv, int total_q, int total_k, int max_q, int max_k, int d, int causal,
               int window_left, float scale, void* stream, int dtype) {
  g_last_error[0] = '\0';
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_UNSUPPORTED, "packed sequences support bf16 and fp16 only (dtype %d)", static_cast<int>(dtype));
  if (B < 0 || Hq < 0 || Hkv < 0 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0 || d < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size (B=%d Hq=%d Hkv=%d total_q=%d total_k=%d max_q=%d max_k=%d d=%d)",
                B, Hq, Hkv, total_q, total_k, max_q, max_k, d);
  if (B == 0 || Hq == 0 || total_q == 0 || max_q == 0) return FA_OK;
  if (Hkv == 0 || Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
  if (window_left < -1) return fail(FA_ERR_INVALID_ARG, "window_left=%d (must be -1 or >= 0)", window_left);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale is not finite");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128)", d);
  if (!q || !k || !v || !o || !cu_q || !cu_k)
    return fail(FA_ERR_INVALID_ARG, "null q/k/v/o/cu_seqlens pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_MISALIGNED, "q, k, v and o must be 16-byte aligned");
  if ((lse && !aligned(lse, 4)) || !aligned(cu_q, 4) || !aligned(cu_k, 4))
    return fail(FA_ERR_MISALIGNED, "lse and cu_seqlens must be 4-byte aligned");
  const uint64_t n_q = (uint64_t)total_q * Hq * d * 2;
  const uint64_t n_kv = (uint64_t)total_k * Hkv * d * 2;
  const uint64_t n_l = (uint64_t)Hq * total_q * sizeof(float);
  if (overlap(o, n_q, q, n_q) || overlap(o, n_q, k, n_kv) || overlap(o, n_q, v, n_kv))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (lse && (overlap(lse, n_l, o, n_q) || overlap(lse, n_l, q, n_q) || overlap(lse, n_l, k, n_kv) ||
              overlap(lse, n_l, v, n_kv)))
    return fail(FA_ERR_INVALID_ARG, "lse overlaps o or an input");
  // one sequence's keys of one head are addressed with 32-bit byte offsets
  if ((uint64_t)max_k * Hkv * d * 2 + (1u << 20) > (uint64_t)INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "max_seqlen_k=%d too long (one sequence's keys must stay below 2 GiB)", max_k);
  const long long rows = fa::mfma_rows_per_workgroup();
  // the launch rounds the (sequence, key/value head) groups up to a multiple of 8
  const long long items = 8 * (((long long)B * Hkv + 7) / 8) * (Hq / Hkv) * ((max_q + rows - 1) / rows);
  if (items > fa::kMaxGridItems) return fail(FA_ERR_UNSUPPORTED, "B*Hq*ceil(max_seqlen_q/%lld) too large", rows);
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = max_q;
  a.d = d;
  a.causal = causal;
  a.window_left = window_left;
  a.scale = scale;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.max_k = max_k;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f16(a, s);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return FA_OK;
}

uint64_t bwd_workspace_bytes(int B, int Hq, int N);

int run_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, float* work, const int* cu_q, const int* cu_k, int B, int Hq,
                   int Hkv, int total_q, int total_k, int max_q, int max_k, int d, int causal, int window_left,
                   float scale, void* stream, int dtype) {
  g_last_error[0] = '\0';
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_UNSUPPORTED, "the backward supports bf16 and fp16 only (dtype %d)", static_cast<int>(dtype));
  if (B < 0 || Hq < 0 || Hkv < 0 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0 || d < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size (B=%d Hq=%d Hkv=%d total_q=%d total_k=%d max_q=%d max_k=%d d=%d)",
                B, Hq, Hkv, total_q, total_k, max_q, max_k, d);
  if (B == 0 || Hq == 0 || total_q == 0 || max_q == 0) return FA_OK;
  if (Hkv == 0 || Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
  if (window_left < -1) return fail(FA_ERR_INVALID_ARG, "window_left=%d (must be -1 or >= 0)", window_left);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale is not finite");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128)", d);
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !work || !cu_q || !cu_k)
    return fail(FA_ERR_INVALID_ARG, "null pointer among q/k/v/o/lse/dout/dq/dk/dv/workspace/cu_seqlens");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(work, 16))
    return fail(FA_ERR_MISALIGNED, "q, k, v, o, dout, dq, dk, dv and the workspace must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(cu_q, 4) || !aligned(cu_k, 4))
    return fail(FA_ERR_MISALIGNED, "lse and cu_seqlens must be 4-byte aligned");
  const uint64_t n_q = (uint64_t)total_q * Hq * d * 2;
  const uint64_t n_kv = (uint64_t)total_k * Hkv * d * 2;
  const uint64_t n_l = (uint64_t)Hq * total_q * sizeof(float);
  const uint64_t n_w = bwd_workspace_bytes(1, Hq, total_q);
  struct Span {
    const void* p;
    uint64_t n;
  };
  const Span outs[4] = {{dq, n_q}, {dk, n_kv}, {dv, n_kv}, {work, n_w}};
  const Span all[10] = {{q, n_q}, {k, n_kv}, {v, n_kv}, {o, n_q}, {lse, n_l}, {dout, n_q},
                        {dq, n_q}, {dk, n_kv}, {dv, n_kv}, {work, n_w}};
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 10; ++j)
      if (j != 6 + i && overlap(outs[i].p, outs[i].n, all[j].p, all[j].n))
        return fail(FA_ERR_INVALID_ARG, "an output (dq, dk, dv or the workspace) overlaps another buffer");
  // one sequence's rows of one head are addressed with 32-bit byte offsets
  if ((uint64_t)max_k * Hkv * d * 2 + (1u << 20) > (uint64_t)INT32_MAX ||
      (uint64_t)max_q * Hq * d * 2 + (1u << 20) > (uint64_t)INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "max_seqlen_q=%d / max_seqlen_k=%d too long (one sequence's rows must stay "
                "below 2 GiB)", max_q, max_k);
  const long long rows = fa::bwd_rows_per_workgroup();
  const long long keys = fa::bwd_keys_per_workgroup(d);
  // the launches round the (sequence, key/value head) groups up to a multiple of 8
  const long long groups8 = 8 * (((long long)B * Hkv + 7) / 8);
  const long long items_q = groups8 * (Hq / Hkv) * ((max_q + rows - 1) / rows);
  const long long items_k = groups8 * ((max_k + keys - 1) / keys);
  if (items_q > fa::kMaxGridItems || items_k > fa::kMaxGridItems || (long long)Hq * total_q / 16 > fa::kMaxGridItems)
    return fail(FA_ERR_UNSUPPORTED, "too many sequences, heads or rows for one launch");
  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.work = work;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = max_q;
  a.d = d;
  a.causal = causal;
  a.window_left = window_left;
  a.scale = scale;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.max_k = max_k;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_bwd_bf16(a, s) : fa::launch_bwd_f16(a, s);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return FA_OK;
}

int run_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale, float v_scale, void* o,
            float* lse, int B, int Hq, int Hkv, int N, int d, int causal, int window_left, float scale,
            void* stream) {
  g_last_error[0] = '\0';
  bool empty;
  if (int st = check_sizes(B, Hq, Hkv, N, d, window_left, scale, FA_DTYPE_BF16, &empty)) return st;
  if (empty) return FA_OK;
  if (!std::isfinite(q_scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale) || !(q_scale > 0.f) ||
      !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(FA_ERR_INVALID_ARG, "the FP8 scales must be finite and > 0 (q %g, k %g, v %g)", (double)q_scale,
                (double)k_scale, (double)v_scale);
  const double c = (double)scale * q_scale * k_scale;
  if (!(std::fabs(c) < 1e30))
    return fail(FA_ERR_INVALID_ARG, "scale * q_scale * k_scale = %g is out of range", c);
  if (!q || !k || !v || !o)
    return fail(FA_ERR_INVALID_ARG, "null q/k/v/o pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_MISALIGNED, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4))
    return fail(FA_ERR_MISALIGNED, "lse must be 4-byte aligned");
  const uint64_t n_q = (uint64_t)B * Hq * N * d;
  const uint64_t n_kv = (uint64_t)B * Hkv * N * d;
  const uint64_t n_o = 2 * n_q;
  if (overlap(o, n_o, q, n_q) || overlap(o, n_o, k, n_kv) || overlap(o, n_o, v, n_kv))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (lse) {
    const uint64_t n_l = (uint64_t)B * Hq * N * sizeof(float);
    if (overlap(lse, n_l, o, n_o) || overlap(lse, n_l, q, n_q) || overlap(lse, n_l, k, n_kv) ||
        overlap(lse, n_l, v, n_kv))
      return fail(FA_ERR_INVALID_ARG, "lse overlaps o or an input");
  }
  if ((uint64_t)N * d + (1u << 20) > (uint64_t)INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "N=%d too long for d=%d (one head must stay below 2 GiB)", N, d);
  const long long rows = fa::fp8_rows_per_workgroup();
  const long long items = (long long)B * Hq * ((N + rows - 1) / rows);
  if (items > fa::kMaxGridItems)
    return fail(FA_ERR_UNSUPPORTED, "B*Hq*ceil(N/%lld)=%lld exceeds one launch", rows, items);
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.causal = causal;
  a.window_left = window_left;
  a.scale = scale;
  const hipError_t e = fa::launch_fwd_fp8(a, q_scale, k_scale, v_scale, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return FA_OK;
}

// ---- key/value cache (decoding) ------------------------------------------

// Splits of each (batch, key/value head, row block)'s key range when the
// caller leaves the choice to the library: about four wavefronts per compute
// unit (one round of the grid; more splits only add merge work and shorter
// streams), at least four 32-key tiles per split, at most 128 splits.
int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  return cus;
}

int auto_splits(long long base_items, int Nk) {
  const int cus = device_cus();
  const long long target = 4LL * cus;
  long long s = base_items > 0 ? (target + base_items - 1) / base_items : 1;
  const long long max_s = std::max(1LL, ((long long)Nk + 32 * 4 - 1) / (32 * 4));
  s = std::min(std::min(s, max_s), 128LL);
  return (int)std::max(1LL, s);
}

// Wavefronts per (batch, key/value head, split): the group's G * Nq rows in
// 32-row blocks, one or two blocks per wavefront.
long long row_items(int Hq, int Hkv, int Nq) {
  const long long rb = ((long long)(Hq / Hkv) * Nq + 31) / 32;
  const int per = fa::decode_row_blocks_per_item((int)std::min<long long>(rb, INT32_MAX));
  return (rb + per - 1) / per;
}

int resolve_splits(int B, int Hq, int Hkv, int Nq, int Nk, int num_splits) {
  if (num_splits > 0) return num_splits;
  return auto_splits((long long)B * Hkv * row_items(Hq, Hkv, Nq), Nk);
}

uint64_t kvcache_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || Hq % Hkv != 0 || num_splits < 0) return 0;
  const int s = resolve_splits(B, Hq, Hkv, Nq, Nk, num_splits);
  return s <= 1 ? 0 : (uint64_t)s * B * Hq * Nq * (uint64_t)(d + 1) * sizeof(float);
}

int run_kvcache(const void* q, const void* k, const void* v, const int* block_table, const int* seqlens, void* o,
                float* lse, float* workspace, int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_pages,
                int page_size, int max_pages, int causal, int window_left, float scale, int num_splits,
                void* stream, int dtype, bool paged, bool use_scratch = false) {
  g_last_error[0] = '\0';
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_UNSUPPORTED, "the key/value-cache path supports bf16 and fp16 only (dtype %d)",
                static_cast<int>(dtype));
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || d < 0 || num_splits < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d splits=%d)", B, Hq, Hkv, Nq,
                Nk, d, num_splits);
  if (paged && (page_size <= 0 || max_pages <= 0 || num_pages <= 0))
    return fail(FA_ERR_INVALID_ARG, "paged cache needs page_size, max_pages_per_seq and num_pages > 0");
  if (B == 0 || Hq == 0 || Nq == 0) return FA_OK;
  if (Hkv == 0 || Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
  if (window_left < -1) return fail(FA_ERR_INVALID_ARG, "window_left=%d (must be -1 or >= 0)", window_left);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale is not finite");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128)", d);
  if (paged && page_size != 16 && page_size % 32 != 0)
    return fail(FA_ERR_UNSUPPORTED, "page_size=%d must be 16 or a multiple of 32", page_size);
  const long long cap = paged ? (long long)page_size * max_pages : (long long)Nk;
  if (cap > INT32_MAX / 2) return fail(FA_ERR_UNSUPPORTED, "cache capacity of %lld keys is too large", cap);
  if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARG, "null q/k/v/o pointer");
  if (paged && (!block_table || !seqlens))
    return fail(FA_ERR_INVALID_ARG, "a paged cache needs block_table and cache_seqlens");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_MISALIGNED, "q, k, v and o must be 16-byte aligned");
  if ((lse && !aligned(lse, 4)) || (seqlens && !aligned(seqlens, 4)) || (block_table && !aligned(block_table, 4)))
    return fail(FA_ERR_MISALIGNED, "lse, cache_seqlens and block_table must be 4-byte aligned");
  // byte offsets inside one head (contiguous) or one page (paged) are 32-bit
  const uint64_t span = paged ? (uint64_t)page_size * Hkv * d * 2 : (uint64_t)Nk * d * 2;
  if (span + (1u << 20) > (uint64_t)INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, paged ? "one page must stay below 2 GiB" : "one head's cache must stay below 2 GiB");
  const int nk = (int)cap;
  if (num_splits > 128) return fail(FA_ERR_UNSUPPORTED, "num_splits=%d (at most 128)", num_splits);
  const int splits = resolve_splits(B, Hq, Hkv, Nq, nk, num_splits);
  if (use_scratch) {
    // the allocation-free form: the library's own scratch array, if it fits
    // (its address is looked up once every other check has passed)
    const uint64_t need = kvcache_workspace_bytes(B, Hq, Hkv, Nq, nk, d, splits);
    if (need > fa::decode_scratch_bytes())
      return fail(FA_ERR_UNSUPPORTED,
                  "%d splits of %lld rows need %llu bytes of scratch, more than the %zu the library holds "
                  "(use fewer splits or fa_fwd_kvcache_paged with a workspace)",
                  splits, (long long)B * Hq * Nq, (unsigned long long)need, fa::decode_scratch_bytes());
  } else if (splits > 1 && !workspace) {
    return fail(FA_ERR_INVALID_ARG, "%d splits need a workspace (fa_fwd_kvcache_workspace_size bytes)", splits);
  }
  if (workspace && !aligned(workspace, 16)) return fail(FA_ERR_MISALIGNED, "the workspace must be 16-byte aligned");
  const uint64_t n_q = (uint64_t)B * Hq * Nq * d * 2;
  const uint64_t n_l = (uint64_t)B * Hq * Nq * sizeof(float);
  const uint64_t n_kv = paged ? (uint64_t)num_pages * page_size * Hkv * d * 2 : (uint64_t)B * Hkv * Nk * d * 2;
  const uint64_t n_w = kvcache_workspace_bytes(B, Hq, Hkv, Nq, nk, d, splits);
  if (overlap(o, n_q, q, n_q) || overlap(o, n_q, k, n_kv) || overlap(o, n_q, v, n_kv))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (lse && (overlap(lse, n_l, o, n_q) || overlap(lse, n_l, q, n_q) || overlap(lse, n_l, k, n_kv) ||
              overlap(lse, n_l, v, n_kv)))
    return fail(FA_ERR_INVALID_ARG, "lse overlaps o or an input");
  if (!use_scratch && splits > 1 && (overlap(workspace, n_w, o, n_q) || overlap(workspace, n_w, q, n_q) ||
                     (lse && overlap(workspace, n_w, lse, n_l)) || overlap(workspace, n_w, k, n_kv) ||
                     overlap(workspace, n_w, v, n_kv)))
    return fail(FA_ERR_INVALID_ARG, "the workspace overlaps another buffer");
  const long long rb = ((long long)(Hq / Hkv) * Nq + 31) / 32;
  if (rb > INT32_MAX / 2) return fail(FA_ERR_UNSUPPORTED, "Hq/Hkv*Nq=%lld query rows per group is too many", 32 * rb);
  const int rb_item = fa::decode_row_blocks_per_item((int)rb);
  const long long row_items = (rb + rb_item - 1) / rb_item;
  const long long items = (long long)B * Hkv * row_items * splits;
  if (items > INT32_MAX / 2) return fail(FA_ERR_UNSUPPORTED, "B*Hkv*row items*splits=%lld is too many", items);
  if (use_scratch) {
    workspace = nullptr;
    if (splits > 1) {
      const hipError_t e = fa::decode_scratch(&workspace);
      if (e != hipSuccess) return fail(FA_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
    }
  }

  fa::DecodeParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.rows = (long long)B * Hq * Nq;
  // workspace: partial outputs [splits][rows][d] (16-byte aligned rows), then
  // partial logsumexps [splits][rows]
  p.part_o = splits > 1 ? workspace : nullptr;
  p.part_lse = splits > 1 ? workspace + (uint64_t)splits * p.rows * d : nullptr;
  p.seqlens = seqlens;
  p.block_table = paged ? block_table : nullptr;
  p.row_stride = paged ? Hkv * d : d;
  p.head_stride = paged ? d : (long long)Nk * d;
  p.batch_stride = paged ? 0 : (long long)Hkv * Nk * d;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = nk;
  p.group = Hq / Hkv;
  p.causal = causal ? 1 : 0;
  // a window of Nk or more keys reaches past key 0 for every row
  p.window_left = window_left >= nk ? -1 : window_left;
  p.n_splits = splits;
  {
    // tiles a row block can need: the whole capacity, or its window plus rows
    long long need = ((long long)nk + 31) / 32;
    if (p.window_left >= 0) need = std::min(need, ((long long)p.window_left + Nq + 31) / 32 + 1);
    p.tiles_per_split = (int)std::max(1LL, (need + splits - 1) / splits);
  }
  p.n_row_blocks = (int)rb;
  p.rb_per_item = rb_item;
  p.n_row_items = (int)row_items;
  p.total_items = (int)items;
  p.page_size = paged ? page_size : 0;
  p.max_pages = paged ? max_pages : 0;
  p.num_pages = paged ? num_pages : 0;
  fa::set_score_scale(p, scale);
  const hipError_t e = fa::launch_decode(p, d, dtype == FA_DTYPE_F16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return FA_OK;
}

uint64_t bwd_workspace_bytes(int B, int Hq, int N) {
  return B <= 0 || Hq <= 0 || N <= 0 ? 0 : 2ull * (uint64_t)B * Hq * N * sizeof(float);
}

int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
            void* dq, void* dk, void* dv, float* work, int B, int Hq, int Hkv, int N, int d, int causal,
            int window_left, float scale, void* stream, int dtype) {
  g_last_error[0] = '\0';
  bool empty;
  if (int st = check_sizes(B, Hq, Hkv, N, d, window_left, scale, dtype, &empty)) return st;
  if (empty) return FA_OK;
  if (dtype == FA_DTYPE_F32)
    return fail(FA_ERR_UNSUPPORTED, "the backward supports bf16 and fp16 only");
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !work)
    return fail(FA_ERR_INVALID_ARG, "null pointer among q/k/v/o/lse/dout/dq/dk/dv/workspace");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(work, 16))
    return fail(FA_ERR_MISALIGNED, "q, k, v, o, dout, dq, dk, dv and the workspace must be 16-byte aligned");
  if (!aligned(lse, 4))
    return fail(FA_ERR_MISALIGNED, "lse must be 4-byte aligned");
  const uint64_t n_q = (uint64_t)B * Hq * N * d * 2;
  const uint64_t n_kv = (uint64_t)B * Hkv * N * d * 2;
  const uint64_t n_l = (uint64_t)B * Hq * N * sizeof(float);
  const uint64_t n_w = bwd_workspace_bytes(B, Hq, N);
  struct Span {
    const void* p;
    uint64_t n;
  };
  const Span outs[4] = {{dq, n_q}, {dk, n_kv}, {dv, n_kv}, {work, n_w}};
  const Span all[10] = {{q, n_q}, {k, n_kv}, {v, n_kv}, {o, n_q}, {lse, n_l}, {dout, n_q},
                        {dq, n_q}, {dk, n_kv}, {dv, n_kv}, {work, n_w}};
  // outs[i] is all[6 + i]; every other buffer must be disjoint from it
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 10; ++j)
      if (j != 6 + i && overlap(outs[i].p, outs[i].n, all[j].p, all[j].n))
        return fail(FA_ERR_INVALID_ARG, "an output (dq, dk, dv or the workspace) overlaps another buffer");
  if ((uint64_t)N * d * 2 + (1u << 20) > (uint64_t)INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "N=%d too long for d=%d (one head must stay below 2 GiB)", N, d);
  const long long rows = fa::bwd_rows_per_workgroup();
  const long long keys = fa::bwd_keys_per_workgroup(d);
  const long long items = (long long)B * Hq * ((N + rows - 1) / rows);
  const long long items_k = (long long)B * Hkv * ((N + keys - 1) / keys);
  if (items > fa::kMaxGridItems || items_k > fa::kMaxGridItems || (long long)B * Hq * N / 16 > fa::kMaxGridItems)
    return fail(FA_ERR_UNSUPPORTED, "B*Hq*N too large for one launch");
  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.work = work;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.causal = causal;
  a.window_left = window_left;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_bwd_bf16(a, s) : fa::launch_bwd_f16(a, s);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
           int N, int d, int causal, int window_left, float scale, void* stream, int dtype) {
  return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream, dtype);
}

int fa_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                int Hkv, int N, int d, int causal, int window_left, float scale, void* stream) {
  return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream, FA_DTYPE_BF16);
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int N, int d, int causal, int window_left, float scale, void* stream) {
  return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream, FA_DTYPE_F16);
}

int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int N, int d, int causal, int window_left, float scale, void* stream) {
  return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream, FA_DTYPE_F32);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                  int max_seqlen_k, int d, int causal, int window_left, float scale, void* stream,
                  int dtype) {
  return run_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k, max_seqlen_q,
                    max_seqlen_k, d, causal, window_left, scale, stream, dtype);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale, float v_scale, void* o,
               float* lse, int B, int Hq, int Hkv, int N, int d, int causal, int window_left, float scale,
               void* stream) {
  return run_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream);
}

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, const int* cache_seqlens, void* o,
                   float* lse, float* workspace, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                   int window_left, float scale, int num_splits, void* stream, int dtype) {
  return run_kvcache(q, k_cache, v_cache, nullptr, cache_seqlens, o, lse, workspace, B, Hq, Hkv, Nq, Nk, d, 0, 0, 0,
                     causal, window_left, scale, num_splits, stream, dtype, false);
}

int fa_fwd_kvcache_paged(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                         const int* cache_seqlens, void* o, float* lse, float* workspace, int B, int Hq, int Hkv,
                         int Nq, int d, int num_pages, int page_size, int max_pages_per_seq, int causal,
                         int window_left, float scale, int num_splits, void* stream, int dtype) {
  return run_kvcache(q, k_pages, v_pages, block_table, cache_seqlens, o, lse, workspace, B, Hq, Hkv, Nq, 0, d,
                     num_pages, page_size, max_pages_per_seq, causal, window_left, scale, num_splits, stream, dtype,
                     true);
}

int fa_fwd_kvcache_paged_noalloc(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                                 const int* cache_seqlens, void* o, float* lse, int B, int Hq, int Hkv, int Nq, int d,
                                 int num_pages, int page_size, int max_pages_per_seq, int causal, int window_left,
                                 float scale, int num_splits, void* stream, int dtype) {
  return run_kvcache(q, k_pages, v_pages, block_table, cache_seqlens, o, lse, nullptr, B, Hq, Hkv, Nq, 0, d,
                     num_pages, page_size, max_pages_per_seq, causal, window_left, scale, num_splits, stream, dtype,
                     true, true);
}

int fa_fwd_kvcache_num_splits(int B, int Hq, int Hkv, int Nq, int Nk) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || Hq % Hkv != 0) return 1;
  return resolve_splits(B, Hq, Hkv, Nq, Nk, 0);
}

int fa_fwd_kvcache_num_splits_for_lengths(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int window_left,
                                          const int* cache_seqlens) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || Hq % Hkv != 0 || window_left < -1 || !cache_seqlens)
    return 1;
  (void)causal;  // the rows' union reaches the last cached key either way
  const int wl = window_left >= Nk ? -1 : window_left;
  // the chunk a split covers is fixed from the capacity (as the launch fixes it)
  long long need = ((long long)Nk + 31) / 32;
  if (wl >= 0) need = std::min(need, ((long long)wl + Nq + 31) / 32 + 1);
  // tiles each sequence's rows need together: keys up to its last one, from
  // the window's left edge for its first row
  std::vector<long long> tiles(B);
  for (int b = 0; b < B; ++b) {
    const long long L = std::min<long long>(std::max(cache_seqlens[b], 0), Nk);
    if (L == 0) {
      tiles[b] = 0;
      continue;
    }
    const long long lo = wl >= 0 ? std::max(0LL, L - Nq - wl) : 0;
    tiles[b] = (L - 1) / 32 + 1 - lo / 32;
  }
  if (*std::max_element(tiles.begin(), tiles.end()) == 0) return 1;  // nothing to read
  const long long rb = row_items(Hq, Hkv, Nq);
  const long long cus = device_cus();
  // Measured on MI355X: about three streaming wavefronts per CU keep HBM
  // busy when each owns one 32-row block, four when each owns two (twice the
  // matrix work per tile), and more than four work items per CU (one-wave
  // workgroups whose LDS stages let four or five share a CU) run in a second
  // round.  Take the fewest splits that give that many streams per CU with
  // at most four items per CU; when no count does both, the most splits
  // within four items per CU.
  const long long two = fa::decode_row_blocks_per_item((int)std::min<long long>(
                            ((long long)(Hq / Hkv) * Nq + 31) / 32, INT32_MAX)) == 2;
  const long long want = (two ? 4 : 3) * cus;
  const long long max_s = std::min(128LL, std::max(1LL, ((long long)Nk + 32 * 4 - 1) / (32 * 4)));
  long long best_fit = 1, best_items = 0;
  for (long long S = 1; S <= max_s; ++S) {
    const long long per = std::max(1LL, (need + S - 1) / S);
    long long chunks = 0;
    for (int b = 0; b < B; ++b) chunks += (tiles[b] + per - 1) / per;
    const long long streams = chunks * Hkv, items = streams * rb;
    if (items <= 4 * cus) {
      if (streams >= want) return (int)S;
      if (items > best_items) {  // more splits that cut no more chunks only add merge work
        best_fit = S;
        best_items = items;
      }
    }
  }
  return (int)best_fit;
}

size_t fa_fwd_kvcache_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
  return (size_t)kvcache_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, int d, int causal,
           int window_left, float scale, void* stream, int dtype) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, causal, window_left, scale,
                 stream, dtype);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* workspace, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                  int causal, int window_left, float scale, void* stream, int dtype) {
  return run_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv,
                        total_q, total_k, max_seqlen_q, max_seqlen_k, d, causal, window_left, scale, stream, dtype);
}

int fa_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, int d, int causal,
                int window_left, float scale, void* stream) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, causal, window_left, scale,
                 stream, FA_DTYPE_BF16);
}

int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, int d, int causal,
               int window_left, float scale, void* stream) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, causal, window_left, scale,
                 stream, FA_DTYPE_F16);
}

size_t fa_bwd_workspace_size(int B, int Hq, int N) { return (size_t)bwd_workspace_bytes(B, Hq, N); }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

const char* fa_last_error(void) { return g_last_error; }

int fa_version(void) { return 500; }  // 0.5.0

}  // extern "C"
