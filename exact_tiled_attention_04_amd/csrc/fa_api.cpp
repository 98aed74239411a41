// C-ABI entry points: argument validation on the host, then the kernel launches.
// The operation, layouts, ownership and error behaviour are specified in
// include/fa.h.
#include "fa.h"

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa_internal.h"

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

size_t elem_size(fa_dtype_t dt) { return dt == FA_DTYPE_F32 ? 4 : 2; }

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Checks shared by the forward and the backward.  Returns FA_OK with
// *empty = true when there is nothing to compute.
int check_sizes(int B, int Hq, int Hkv, int N, int d, int window_left, float scale, fa_dtype_t dtype,
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
  if (!(scale > 0.f))
    return fail(FA_ERR_UNSUPPORTED, "scale=%g: only positive scales are supported", (double)scale);
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128)", d);
  return FA_OK;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
        int N, int d, int causal, int window_left, float scale, void* stream, fa_dtype_t dtype) {
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
  if (!(c < 1e30))
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

uint64_t bwd_workspace_bytes(int B, int Hq, int N) {
  return B <= 0 || Hq <= 0 || N <= 0 ? 0 : 2ull * (uint64_t)B * Hq * N * sizeof(float);
}

int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
            void* dq, void* dk, void* dv, float* work, int B, int Hq, int Hkv, int N, int d, int causal,
            int window_left, float scale, void* stream, fa_dtype_t dtype) {
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
  const long long items = (long long)B * Hq * ((N + rows - 1) / rows);
  if (items > fa::kMaxGridItems || (long long)B * Hq * N / 16 > fa::kMaxGridItems)
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
           int N, int d, int causal, int window_left, float scale, void* stream, fa_dtype_t dtype) {
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

int fa_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale, float v_scale, void* o,
               float* lse, int B, int Hq, int Hkv, int N, int d, int causal, int window_left, float scale,
               void* stream) {
  return run_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, window_left, scale, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, int d, int causal,
           int window_left, float scale, void* stream, fa_dtype_t dtype) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, causal, window_left, scale,
                 stream, dtype);
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

int fa_version(void) { return 300; }  // 0.3.0

}  // extern "C"
