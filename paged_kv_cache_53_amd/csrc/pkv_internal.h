// Internal declarations shared by the HIP sources of libpagedkv (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// ---------------------------------------------------------------- launch parameters
struct ScatterArgs {
  const void* k;
  const void* v;
  const int64_t* slot_mapping;
  void* k_pool;
  void* v_pool;
  int64_t k_stride;      // elements between consecutive tokens of k
  int64_t v_stride;
  int32_t num_tokens;
  int32_t num_blocks;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block_size;
};

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  // workspace views
  int32_t* counters;     // [0] = number of (row, partition) units, [1] = units handed out by claim
                         // after the ones the waves of the persistent grid take in fixed rounds
  int4* units;           // per (row, partition) pair, largest first: {row, partition, row length,
                         // block id of the partition's first block}
  float* part_m;         // [S][Hq][max_parts]  running max of x*log2(e)
  float* part_l;         // [S][Hq][max_parts]  sum of weights
  float* part_acc;       // [S][Hq][max_parts][D]  unnormalised weighted V
  int32_t bt_stride;
  int32_t num_seqs;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t group;         // n_q_heads / n_kv_heads
  int32_t num_blocks;
  int32_t block_size;
  int32_t log2_block;
  int32_t max_seq_len;
  int32_t part_tokens;   // partition size in tokens (multiple of 32)
  int32_t max_parts;
  int32_t out_f32;       // 1: out is float, 0: out has the KV type
  float scale_log2;      // scale * log2(e) (times the key scale of a quantised cache): scores
                         // are kept in the base-2 domain
  float v_scale;         // value scale of a quantised cache (1 otherwise)
  int32_t flat_bps;      // > 0: flat spans of this many blocks, block_tables holds one span per row
  int32_t cache_tokens;  // per-tile load policy: tiles starting before this token of their row are read
                         // cacheable, the others streamed
};

// How the decode kernel reads the pools: every tile cacheable, every tile streamed (non-temporal), or
// per tile (cacheable below DecodeArgs::cache_tokens).
enum LoadPolicy { kLoadCached = 0, kLoadStreamed = 1, kLoadMixed = 2 };

// The fused decode step's own arguments (beyond the scatter's and the decode's).
struct StepArgs {
  const int64_t* slots;   // one slot per batch row, at an address the kernel can read
  int32_t* block_tables;  // the decode's tables and lengths, which the step's append updates
  int32_t* seq_lens;
  float k_scale;          // FP8 pools: the scatter stores codes of x / scale
  float v_scale;
};

// Workspace carve-up shared by the size query and the launcher.
struct WorkspaceLayout {
  size_t counters_off, units_off, m_off, l_off, acc_off, total;
};
WorkspaceLayout workspace_layout(int32_t num_seqs, int32_t n_q_heads, int32_t head_dim,
                                 int32_t max_parts);
int32_t partition_tokens(int32_t max_seq_len, int32_t partition_size);

// ---------------------------------------------------------------- launchers (return hipError_t)
hipError_t launch_reshape_and_cache(const ScatterArgs& a, int dtype, hipStream_t stream);
// The scatter into an FP8 E4M3 cache: sources of src_dtype, codes of x / scale.
hipError_t launch_reshape_and_cache_fp8(const ScatterArgs& a, int src_dtype, float k_scale, float v_scale,
                                        hipStream_t stream);
// Copies whole blocks (both pools, every head) for each (src, dst) pair.
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n_pairs,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t stream);
// Copies whole blocks (both pools) from one block array to another (device or pinned host memory).
hipError_t launch_move_blocks(const void* src_k, const void* src_v, int32_t src_blocks, void* dst_k, void* dst_v,
                              int32_t dst_blocks, const int32_t* pairs, int32_t n_pairs, int64_t block_bytes,
                              hipStream_t stream);
hipError_t launch_append_slots(const int64_t* slot_mapping, int32_t num_seqs, int32_t* block_tables,
                               int32_t stride, int32_t* seq_lens, int32_t block_size,
                               hipStream_t stream);
hipError_t launch_decode_plan(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);
// Counts out-of-pool block-table entries among each row's first ceil(L / B) (result: {count, first row}).
hipError_t launch_check_tables(const int32_t* tables, int32_t stride, const int32_t* seq_lens, int32_t num_seqs,
                               int32_t block_size, int32_t num_blocks, int32_t max_seq_len, int32_t* result,
                               hipStream_t stream);
// The fused step's first kernel: append, scatter (sc.num_tokens == a.num_seqs tokens, rows of
// dtype; kv_fp8: quantised pools) and plan.  head_dim must be 64 or 128.
hipError_t launch_step_prologue(const DecodeArgs& a, const ScatterArgs& sc, const StepArgs& st, int dtype,
                                bool kv_fp8, int head_dim, hipStream_t stream);
// dtype: the type of q and of the results; kv_fp8: the pools hold FP8 E4M3 codes (else dtype)
// path: 0 = vector, 1 = MFMA; pol: a LoadPolicy
hipError_t launch_decode_main(const DecodeArgs& a, int dtype, bool kv_fp8, int head_dim, int path, int pol,
                              int32_t grid, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);
// Persistent grid size for the main decode kernel on the current device.
hipError_t decode_main_grid_cap(int dtype, bool kv_fp8, bool flat, int head_dim, int path, int group,
                                int block_size, int pol, int32_t* cap);

// Physical memory of a flat-span pool is mapped in chunks of this size unless the caller picks another.
constexpr size_t PKV_SPAN_DEFAULT_CHUNK = size_t{2} << 20;

// ---------------------------------------------------------------- timing hooks
void timing_before(int kernel, hipStream_t stream);
void timing_after(int kernel, hipStream_t stream);

}  // namespace pkv
