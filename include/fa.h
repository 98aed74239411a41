/*
 * fa.h -- exact attention forward and backward for AMD MI355X (gfx950), C ABI.
 *
 * Operation (one call):  for every batch b, query head h and query row i,
 *
 *     s_ij   = scale * sum_c q[b][h][i][c] * k[b][g(h)][j][c]
 *     s_ij   = -inf                       where (i, j) is masked
 *     o[b][h][i][:] = sum_j softmax_j(s_i.) * v[b][g(h)][j][:]
 *     lse[b][h][i]  = log( sum_j exp(s_ij) )          (natural log)
 *
 * with g(h) = h / (Hq / Hkv) (consecutive groups of query heads share one
 * key/value head) and (i, j) masked when (causal && j > i) or
 * (window_left >= 0 && j < i - window_left).
 *
 * This is standard attention, softmax(Q K^T) V, as drawn in the "AS-IS"
 * diagram of the Flash Attention page (heepie.pages.dev), computed the IO-aware
 * way of that page's "TO-BE" diagram and tiling section: K/V tiles are staged
 * on chip, the N x N score matrix never reaches device memory, and an online
 * softmax (FlashAttention quiz, question 4) rescales a running partial result.
 * The mask and the GQA head sharing follow the Hacker News answer on GQA and
 * sliding windows (a window only changes the mask; GQA only changes which K/V
 * head a query head reads).  The scale, the causal convention (key j visible
 * to query i iff j <= i), the window convention (window_left keys before the
 * query stay visible, plus the query's own key) and the logsumexp output are
 * this library's readings of points the pages leave open.
 *
 * Layout (all contiguous, row-major, element type given by the dtype):
 *     q, o : [B][Hq][N][d]          k, v : [B][Hkv][N][d]
 *     lse  : [B][Hq][N] float32
 * o has the element type of q.  d is the fastest axis.
 *
 * Ownership and execution:
 *   - Every pointer is device memory on the current HIP device, allocated and
 *     owned by the caller.  q, k and v are only read and may alias each other;
 *     o and lse are only written and must not overlap any input or each other.
 *   - The library allocates no device memory and keeps no per-call state; all
 *     entry points are thread-safe.
 *   - The call is asynchronous: it validates its arguments on the host,
 *     enqueues the work on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns.  It never synchronises.  Faults inside the kernel surface at
 *     the caller's next synchronisation, as for any HIP launch.
 *   - Results are deterministic: the same inputs give bit-identical o and lse.
 *
 * Errors: every argument is checked on the host before anything is enqueued;
 * on failure the call returns a negative fa_status_t, writes nothing, and
 * fa_last_error() (thread-local) describes the problem.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  Entry points take the type as a plain int holding one of
 * these values (any other int is rejected with FA_ERR_UNSUPPORTED). */
typedef enum {
  FA_DTYPE_F32 = 0,   /* IEEE binary32 */
  FA_DTYPE_F16 = 1,   /* IEEE binary16 */
  FA_DTYPE_BF16 = 2   /* bfloat16 */
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, negative size, Hq % Hkv != 0,
                              window_left < -1, non-finite scale          */
  FA_ERR_UNSUPPORTED = -2, /* d not 64 or 128, unknown dtype, one head's
                              K or V of 2 GiB or more                     */
  FA_ERR_MISALIGNED = -3,  /* q, k, v or o not 16-byte aligned, lse not
                              4-byte aligned                              */
  FA_ERR_HIP = -4          /* the HIP runtime reported an error at launch */
} fa_status_t;

/*
 * Attention forward for element type `dtype`.
 *
 *   q, k, v      inputs (device), layouts above.
 *   o            output (device), same element type and layout as q.
 *   lse          output (device) float32 [B][Hq][N], or NULL to skip it.
 *   B, Hq, Hkv   batch size, query heads, key/value heads (Hq % Hkv == 0).
 *   N            sequence length (queries and keys alike).
 *   d            head dimension: 64 or 128.
 *   causal       nonzero: key j is hidden from query i when j > i.
 *   window_left  -1: no window.  >= 0: key j is hidden from query i when
 *                j < i - window_left.  Composes with `causal`.
 *   scale        multiplier on q.k before the softmax; any finite value
 *                (the usual one is 1/sqrt(d); a negative scale favours
 *                dissimilar keys, zero gives the mean of the visible V rows).
 *   stream       hipStream_t to enqueue on, NULL for the null stream.
 *
 * If B, Hq or N is 0 the call does nothing and returns FA_OK (pointers are
 * then not inspected).  Otherwise Hkv must be >= 1.
 * Returns FA_OK or a negative fa_status_t.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int Hq, int Hkv, int N, int d, int causal, int window_left,
           float scale, void *stream, int dtype);

/* The same operation with the element type fixed by the name. */
int fa_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                int B, int Hq, int Hkv, int N, int d, int causal, int window_left,
                float scale, void *stream);
int fa_fwd_f16(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, int causal, int window_left,
               float scale, void *stream);
int fa_fwd_f32(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, int causal, int window_left,
               float scale, void *stream);

/*
 * Attention forward over a batch of sequences of different lengths, packed.
 *
 * Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and
 * key/value rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v; with
 * Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] and Lk likewise, its query row i
 * stands at key position Lk - Lq + i (equal lengths: ordinary self-attention,
 * fewer queries than keys: the queries are the sequence's last tokens), and
 * the operation is fa_fwd's within each sequence, the causal mask and window
 * measured from that position.  Rows that see no key (Lq > Lk under a causal
 * mask) get o = 0 and lse = -inf.  Variable-length attention is a title on the
 * pages (FlashMask, PagedAttention in the FlashAttention-2 (PL) literature);
 * the packing and the alignment are this library's readings.
 *
 *   q, o          [total_q][Hq][d] (token-major), element type dtype (BF16/F16).
 *   k, v          [total_k][Hkv][d].
 *   lse           [Hq][total_q] float32 (natural log), or NULL.
 *   cu_seqlens_q, cu_seqlens_k  device int32 [B+1], nondecreasing, from 0 to
 *                 total_q / total_k (the kernel clamps them into range, so
 *                 inconsistent offsets give unspecified values, never an
 *                 access outside the tensors).
 *   max_seqlen_q, max_seqlen_k  upper bounds of Lq and Lk over the batch
 *                 (a smaller value leaves a longer sequence's query rows from
 *                 max_seqlen_q on unwritten and its other rows unspecified,
 *                 never an access outside the tensors).
 *   B, Hq, Hkv, d, causal, window_left, scale, stream  as for fa_fwd.
 *
 * Rows of o and lse that no sequence owns (from cu_seqlens_q[B] to total_q)
 * are left exactly as the caller passed them: the call writes only the rows
 * of the sequences.
 *
 * Errors as for fa_fwd; FA_DTYPE_F32 is FA_ERR_UNSUPPORTED; max_seqlen_k * Hkv
 * * d * 2 bytes must stay below 2 GiB.
 */
int fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int *cu_seqlens_q, const int *cu_seqlens_k, int B, int Hq, int Hkv,
                  int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                  int causal, int window_left, float scale, void *stream, int dtype);

/*
 * Attention forward on FP8 inputs with per-tensor scales.
 *
 * The FlashAttention quiz (question 6) and the FlashAttention-2 (PL) article
 * (section "FlashAttention-3") name 8-bit floating point, with its rounding
 * error kept in check, as a further speed-up.  Here q, k and v hold OCP E4M3
 * bytes (bias 7, 3 mantissa bits, largest finite 448, no infinities; the
 * torch.float8_e4m3fn encoding) and each tensor has one float32 scale: an
 * element stands for e4m3(byte) * x_scale.  The operation is fa_fwd's on those
 * values, with
 *
 *     s_ij = scale * q_scale * k_scale * sum_c e4m3(q_ic) * e4m3(k_jc)
 *     o    = v_scale * sum_j softmax_j(s_i.) * e4m3(v_j)
 *
 * Both products run on the FP8 matrix cores and accumulate in fp32; the
 * probabilities are rounded to E4M3 for the second product (the row sum is
 * taken before that rounding), so o carries an error of at most about 2^-4
 * of sum_j p_ij |v_j|, plus the rounding of o to bfloat16.
 *
 *   q, k, v      E4M3 bytes (device), layouts above with 1-byte elements.
 *                The NaN bytes 0x7f and 0xff are not valid inputs: rows whose
 *                key tiles hold one may come out NaN.
 *   q_scale, k_scale, v_scale
 *                per-tensor dequantisation scales, finite and > 0.
 *   o            output (device), bfloat16, layout of q.
 *   lse          output (device) float32 [B][Hq][N] (natural log of the sum
 *                of exp(s_ij) over visible keys), or NULL to skip it.
 *   B ... stream as for fa_fwd.
 *
 * Errors and ownership as for fa_fwd; in addition a scale that is not finite
 * and positive, or whose product with scale overflows, is FA_ERR_INVALID_ARG.
 */
int fa_fwd_fp8(const void *q, const void *k, const void *v,
               float q_scale, float k_scale, float v_scale, void *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, int causal, int window_left,
               float scale, void *stream);

/*
 * Attention of a few query rows against a key/value cache (decoding).
 *
 * Batch b has a cache of L_b = cache_seqlens[b] keys (all Nk when
 * cache_seqlens is NULL) and Nq query rows that stand at the end of it: row i
 * is position L_b - Nq + i of the sequence.  For query head h (key/value head
 * g(h) as in fa_fwd), row i and cached key j < L_b,
 *
 *     s_ij = scale * sum_c q[b][h][i][c] * k[b][g(h)][j][c]
 *     (i, j) masked when (causal && j > L_b - Nq + i) or
 *                        (window_left >= 0 && j < L_b - Nq + i - window_left)
 *     o[b][h][i][:] = sum_j softmax_j(s_i.) v[b][g(h)][j][:],  lse = log sum_j exp(s_ij)
 *
 * i.e. the last Nq rows of fa_fwd over the whole sequence (the causal mask
 * aligned to the end of the cache).  A row that sees no key (L_b < Nq - i
 * under a causal mask, or L_b = 0) gets o = 0 and lse = -inf.  The pages
 * name decoding and inference only in passing (the Hacker News thread, the
 * FastAttention abstract); the alignment, the lengths and the empty-row
 * values are this library's readings.
 *
 * The key range of each (batch, key/value head) is cut into num_splits parts
 * processed in parallel; each writes a partial output and its logsumexp to
 * the workspace, and a second kernel merges them (lse = log sum_s exp(lse_s),
 * o = sum_s exp(lse_s - lse) o_s), the identity the tiling section of the
 * Flash Attention page rests on.  num_splits = 0 lets the library choose
 * (fa_fwd_kvcache_num_splits); with one split nothing goes through the
 * workspace.  Results are deterministic for a given num_splits.
 *
 *   q             [B][Hq][Nq][d], element type dtype (FA_DTYPE_BF16 or F16).
 *   k_cache, v_cache  [B][Hkv][Nk][d], same element type; keys at or past a
 *                 batch's length are never read.
 *   cache_seqlens device int32 [B] in [0, Nk] (values outside are clamped), or
 *                 NULL for Nk everywhere.
 *   o             [B][Hq][Nq][d] output, element type dtype.
 *   lse           [B][Hq][Nq] float32 output (natural log), or NULL.
 *   workspace     device memory of fa_fwd_kvcache_workspace_size(B, Hq, Hkv,
 *                 Nq, Nk, d, num_splits) bytes, 16-byte aligned (NULL allowed
 *                 when that size is 0); contents on entry ignored, on return
 *                 unspecified.
 *   B, Hq, Hkv, d, causal, window_left, scale, stream  as for fa_fwd.
 *   Nq            query rows per sequence; Nk cache capacity in keys.
 *   num_splits    0..128 (0: the library's choice).
 *
 * o, lse and the workspace must not overlap each other or any input.
 * Errors as for fa_fwd, plus FA_ERR_UNSUPPORTED for FA_DTYPE_F32 and
 * FA_ERR_INVALID_ARG for a missing workspace when more than one split runs.
 */
int fa_fwd_kvcache(const void *q, const void *k_cache, const void *v_cache,
                   const int *cache_seqlens, void *o, float *lse, float *workspace,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                   int window_left, float scale, int num_splits, void *stream,
                   int dtype);

/*
 * The same operation on a paged cache: the keys of batch b are spread over
 * fixed-size pages, key j living in page block_table[b][j / page_size] at
 * slot j % page_size.
 *
 *   k_pages, v_pages  [num_pages][page_size][Hkv][d] (token-major pages).
 *   block_table   device int32 [B][max_pages_per_seq] page indices; entries
 *                 past a batch's length are not read; an index outside
 *                 [0, num_pages) reads as zeros (never out of bounds).
 *   cache_seqlens device int32 [B], required, in [0, page_size *
 *                 max_pages_per_seq] (clamped).
 *   page_size     16 or a multiple of 32.
 *   Everything else as fa_fwd_kvcache, with Nk = page_size * max_pages_per_seq
 *   for the workspace size.
 */
int fa_fwd_kvcache_paged(const void *q, const void *k_pages, const void *v_pages,
                         const int *block_table, const int *cache_seqlens, void *o,
                         float *lse, float *workspace, int B, int Hq, int Hkv, int Nq,
                         int d, int num_pages, int page_size, int max_pages_per_seq,
                         int causal, int window_left, float scale, int num_splits,
                         void *stream, int dtype);

/*
 * fa_fwd_kvcache_paged without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The splits' partial outputs and
 * logsumexps go to a scratch array the library holds in device memory, 16 MiB
 * per GPU (one copy on each GPU it runs on, held until the process ends), so
 * splits * B * Hq * Nq * (d + 1) * 4 bytes must not exceed 16 MiB (with one
 * split no scratch is used); a larger request returns FA_ERR_UNSUPPORTED and
 * enqueues nothing.  The call allocates nothing.  Every slot of the scratch
 * a call reads is written earlier in the same call, so nothing needs
 * clearing; but all calls on one GPU share the array, so calls that can
 * overlap on one GPU (different streams, no ordering between them) race and
 * must not be issued.  Arguments, results and other errors as for
 * fa_fwd_kvcache_paged; the first call on a device also looks up the
 * array's address there (a failure is FA_ERR_HIP).
 */
int fa_fwd_kvcache_paged_noalloc(const void *q, const void *k_pages, const void *v_pages,
                                 const int *block_table, const int *cache_seqlens, void *o,
                                 float *lse, int B, int Hq, int Hkv, int Nq, int d, int num_pages,
                                 int page_size, int max_pages_per_seq, int causal, int window_left,
                                 float scale, int num_splits, void *stream, int dtype);

/* Splits fa_fwd_kvcache uses when num_splits = 0 (enough parallel work for
 * the current device, at least four 32-key tiles per split); 1 for sizes
 * that compute nothing. */
int fa_fwd_kvcache_num_splits(int B, int Hq, int Hkv, int Nq, int Nk);

/* A split count for caches whose lengths the caller knows on the host
 * (cache_seqlens_host: B lengths, read here only; pass the result as
 * num_splits together with the same lengths on the device).  Since a split
 * covers a fixed share of the capacity, short sequences leave their last
 * splits empty; this counts the splits that will read keys and takes the
 * fewest that give about three streaming wavefronts per compute unit (four
 * when a GQA group's G * Nq query rows make an even number, at least four,
 * of 32-row blocks, so that one wavefront takes two of them) while keeping
 * every work item in one wave of the
 * grid (at most four per unit), else the fewest splits that put the most
 * work items in that wave; at least four 32-key tiles per split and at most
 * 128.  Equal full lengths give fewer splits than fa_fwd_kvcache_num_splits
 * when three streams per unit already suffice.
 * Returns 1 for sizes that compute nothing or a null pointer. */
int fa_fwd_kvcache_num_splits_for_lengths(int B, int Hq, int Hkv, int Nq, int Nk, int causal,
                                          int window_left, const int *cache_seqlens_host);

/* Workspace bytes fa_fwd_kvcache(_paged) needs for these sizes and
 * num_splits (0 = the library's choice): splits * B * Hq * Nq * (d + 1) *
 * sizeof(float) when more than one split runs, else 0. */
size_t fa_fwd_kvcache_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);

/*
 * Gradients of fa_fwd's output with respect to q, k and v.
 *
 * For an upstream gradient dout = dL/do (the logsumexp output is taken to
 * carry no gradient), with P the forward's probabilities (masked pairs 0):
 *
 *     dv[b][g]    = sum over the query heads h of group g of  P^T dout[b][h]
 *     dP          = dout V^T
 *     dS          = P * (dP - D),   D_i = sum_c dout_ic * o_ic
 *     dq[b][h]    = scale * dS K
 *     dk[b][g]    = sum over the query heads h of group g of  scale * dS^T q[b][h]
 *
 * This is the derivative of the operation above (the pages give no backward
 * formulas).  P is recomputed from q, k and the saved lse instead of being
 * stored, the trade of extra FLOPs for less memory traffic that the Flash
 * Attention page (heepie.pages.dev, tiling section) describes.
 *
 *   q, k, v      the forward's inputs (device), layouts above.
 *   o, lse       the forward's outputs for these inputs (lse is required).
 *   dout         upstream gradient, same element type and layout as o.
 *   dq, dk, dv   outputs (device), element type of q, layouts of q, k, v.
 *   workspace    device memory of fa_bwd_workspace_size(B, Hq, N) bytes,
 *                16-byte aligned, owned by the caller; its contents on entry
 *                are ignored and on return are unspecified.
 *   B ... stream as for fa_fwd.  dtype: FA_DTYPE_BF16 or FA_DTYPE_F16
 *                (FA_DTYPE_F32 returns FA_ERR_UNSUPPORTED).
 *
 * dq, dk, dv and the workspace must not overlap each other or any input.
 * The library allocates nothing; the call is asynchronous on `stream` (three
 * kernel launches) and bit-reproducible (no atomics: each key/value head's
 * dk and dv are summed over its query heads inside one workgroup).  Errors
 * are reported as for fa_fwd; nothing is written on failure.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
           const void *dout, void *dq, void *dk, void *dv, float *workspace,
           int B, int Hq, int Hkv, int N, int d, int causal, int window_left,
           float scale, void *stream, int dtype);
int fa_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                const void *dout, void *dq, void *dk, void *dv, float *workspace,
                int B, int Hq, int Hkv, int N, int d, int causal, int window_left,
                float scale, void *stream);
int fa_bwd_f16(const void *q, const void *k, const void *v, const void *o, const float *lse,
               const void *dout, void *dq, void *dk, void *dv, float *workspace,
               int B, int Hq, int Hkv, int N, int d, int causal, int window_left,
               float scale, void *stream);

/*
 * Gradients of fa_fwd_varlen's output: the fa_bwd operation within each
 * packed sequence, with fa_fwd_varlen's layouts, offsets and alignment (query
 * row i of sequence b at key position Lk - Lq + i; the causal mask and window
 * measured from there).
 *
 *   q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q,
 *   total_k, max_seqlen_q, max_seqlen_k, d, causal, window_left, scale
 *                as given to (and returned by) fa_fwd_varlen; lse is
 *                required.  Rows that saw no key (lse = -inf) pass no
 *                gradient.
 *   dout         [total_q][Hq][d], element type of q.
 *   dq           [total_q][Hq][d]; dk, dv [total_k][Hkv][d].  Rows of every
 *                sequence up to max_seqlen_q queries and max_seqlen_k keys are
 *                written (keys no query sees get 0); rows outside every
 *                sequence are left as they were.
 *   workspace    device memory of fa_bwd_workspace_size(1, Hq, total_q)
 *                bytes, 16-byte aligned, as for fa_bwd.
 *   stream, dtype  as for fa_bwd.
 *
 * Offsets are clamped into range as in fa_fwd_varlen, so inconsistent ones
 * give unspecified values, never an access outside the tensors.  Overlap
 * rules, errors, reproducibility and ownership as for fa_bwd; one sequence's
 * rows of all heads must stay below 2 GiB (max_seqlen * H * d * 2 bytes).
 */
int fa_bwd_varlen(const void *q, const void *k, const void *v, const void *o, const float *lse,
                  const void *dout, void *dq, void *dk, void *dv, float *workspace,
                  const int *cu_seqlens_q, const int *cu_seqlens_k, int B, int Hq, int Hkv,
                  int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                  int causal, int window_left, float scale, void *stream, int dtype);

/* Bytes of workspace fa_bwd needs: 2 * B * Hq * N * sizeof(float) (0 when
 * any size is 0 or negative); fa_bwd_varlen takes B = 1, N = total_q. */
size_t fa_bwd_workspace_size(int B, int Hq, int N);

/* Static, human-readable name of a status code (never NULL). */
const char *fa_status_string(int status);

/* Detail of this thread's last failing call ("" if none).  The pointer stays
 * valid until this thread's next call into the library. */
const char *fa_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
