// Kernel parameters of attention against a key/value cache (decoding),
// shared by the C-ABI wrapper and the decoding kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Attention of Nq query rows against a key/value cache (decoding): kernel
// parameters, validated and derived on the host.
struct DecodeParams {
  const void* q;            // [B][Hq][Nq][d]
  const void* k;            // contiguous [B][Hkv][Nk][d], or pages [num_pages][page_size][Hkv][d]
  const void* v;
  void* o;                  // [B][Hq][Nq][d]
  float* lse;               // [B][Hq][Nq] or null
  float* part_o;            // [n_splits][rows][d] (n_splits > 1)
  float* part_lse;          // [n_splits][rows]
  const int* seqlens;       // [B] cache lengths, or null (every length Nk)
  const int* block_table;   // [B][max_pages] page indices (paged cache), else null
  long long rows;           // B * Hq * Nq
  long long batch_stride;   // contiguous cache: elements between batches
  long long head_stride;    // contiguous cache: elements between key/value heads
  int row_stride;           // elements between consecutive keys of one head
  int B, Hq, Hkv, Nq, Nk;   // Nk: cache capacity in keys (paged: page_size * max_pages)
  int group;                // Hq / Hkv
  int causal;
  int window_left;          // -1 = none
  int n_splits;             // splits of each key range (1: o and lse written directly)
  int tiles_per_split;      // 32-key tiles per split, from the capacity (or window) and n_splits
  int n_row_blocks;         // ceil(group * Nq / 32)
  int rb_per_item;          // 32-row blocks one wavefront owns (decode_row_blocks_per_item)
  int n_row_items;          // ceil(n_row_blocks / rb_per_item)
  int total_items;          // B * Hkv * n_row_items * n_splits (one wavefront each)
  int page_size, max_pages, num_pages;
  float scale_log2;         // |scale| * log2(e) (log2(e) for a zero scale)
  int q_sign;               // sign of the scale, applied to the query registers (as FwdParams)
};

hipError_t launch_decode(const DecodeParams& p, int d, bool f16, hipStream_t stream);
// How many 32-row blocks of a GQA group one wavefront takes (1 or 2): two
// blocks share every K and V tile read into LDS.
int decode_row_blocks_per_item(int n_row_blocks);
int decode_waves_per_workgroup();
// The allocation-free entry point's scratch: its size in bytes, and its device
// address on the current device (looked up once per device).
size_t decode_scratch_bytes();
hipError_t decode_scratch(float** ptr);

}  // namespace fa
