// Slot-mapping scatter and the device half of the on-demand block append.
//
// reshape_and_cache writes every new token's key and value rows into the
// physical slot the block manager gave it ("PagedAttention -- Math + Memory
// Model", section "PagedAttention: blocks and the block table"); it copies
// bits, never converts.  reshape_and_cache_fp8 is the same scatter into a
// quantised cache (codes of x / scale).  Four threads move one 16-byte key
// vector and the matching value elements; the per-thread bodies are shared
// with the fused decode-step prologue (scatter_body.h).
// append_slots records, per batch row, the block of the new token's slot in
// the row's block table and bumps the row's length.  copy_blocks makes the
// private copies of shared blocks that copy-on-write appends ask for.
#include <algorithm>

#include "scatter_body.h"

namespace pkv {
namespace {

// Thread gid -> (token t, head h, vector c, quarter sub) of a scatter with C vectors per head row.
struct ScatterItem {
  int t, h, c, sub;
};
__device__ inline bool scatter_item(const ScatterArgs& a, int C, ScatterItem& it) {
  const int64_t per_token = static_cast<int64_t>(a.n_kv_heads) * C;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= 4 * per_token * a.num_tokens) return false;
  const int64_t item = gid >> 2;
  it.sub = static_cast<int>(gid & 3);
  it.t = static_cast<int>(item / per_token);
  const int rem = static_cast<int>(item - static_cast<int64_t>(it.t) * per_token);
  it.h = rem / C;
  it.c = rem - it.h * C;
  return true;
}

template <typename E>  // E: uint32_t (fp32) or uint16_t (fp16/bf16) -- raw bits
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ScatterArgs a) {
  ScatterItem it;
  if (!scatter_item(a, a.head_dim / (16 / static_cast<int>(sizeof(E))), it)) return;
  scatter_quarter<E>(a, it.t, it.h, it.c, it.sub, a.slot_mapping[it.t]);
}

// Four threads per 16-element key vector of one (token, head) and the 16 matching value elements.
template <typename S>  // source element type: float, _Float16 or __bf16
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(ScatterArgs a, float k_scale, float v_scale) {
  ScatterItem it;
  if (!scatter_item(a, a.head_dim / 16, it)) return;
  scatter_quarter_fp8<S>(a, it.t, it.h, it.c, it.sub, a.slot_mapping[it.t], k_scale, v_scale);
}

__global__ __launch_bounds__(256) void append_slots_kernel(const int64_t* __restrict__ slot_mapping,
                                                           int32_t num_seqs, int32_t* block_tables,
                                                           int32_t stride, int32_t* seq_lens,
                                                           int32_t block_size) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= num_seqs) return;
  append_row(slot_mapping[i], block_tables, stride, seq_lens, block_size, i);
}

// Block copies between two block arrays (the same pool for copy-on-write; a device pool and host
// swap space for swapping): block dst of the destination becomes a copy of block src of the source.
// Grid: (pair, pool, slice); each workgroup moves one slice of one block with 16-byte loads and
// stores.  Either array may be pinned host memory, reached over the host link.
__global__ __launch_bounds__(256) void move_blocks_kernel(const void* src_k, const void* src_v, void* dst_k,
                                                          void* dst_v, const int32_t* pairs, int32_t src_blocks,
                                                          int32_t dst_blocks, int64_t block_bytes) {
  const int src = pairs[2 * static_cast<int64_t>(blockIdx.x)];
  const int dst = pairs[2 * static_cast<int64_t>(blockIdx.x) + 1];
  if (src < 0 || dst < 0 || src >= src_blocks || dst >= dst_blocks) return;
  if (src == dst && (blockIdx.y ? src_v == dst_v : src_k == dst_k)) return;   // a block onto itself
  const char* sp = static_cast<const char*>(blockIdx.y ? src_v : src_k);
  char* dp = static_cast<char*>(blockIdx.y ? dst_v : dst_k);
  const uint4* s = reinterpret_cast<const uint4*>(sp + src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>(dp + dst * block_bytes);
  const int64_t vecs = block_bytes / 16;
  for (int64_t i = static_cast<int64_t>(blockIdx.z) * blockDim.x + threadIdx.x; i < vecs;
       i += static_cast<int64_t>(gridDim.z) * blockDim.x)
    d[i] = s[i];
}

// Counts block-table entries outside [0, num_blocks) among each row's first ceil(L / B) entries
// (L: the row's length, clamped to [0, max_seq_len] as decode clamps it).  One workgroup per row;
// result[0] += bad entries, result[1] = min(result[1], first row with one).  Plain vector atomics.
__global__ __launch_bounds__(256) void check_tables_kernel(const int32_t* __restrict__ tables, int32_t stride,
                                                           const int32_t* __restrict__ seq_lens, int32_t block_size,
                                                           int32_t num_blocks, int32_t max_seq_len,
                                                           int32_t* result) {
  const int s = blockIdx.x;
  int L = seq_lens[s];
  L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
  const int nb = (L + block_size - 1) / block_size;
  int bad = 0;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) {
    const int id = tables[static_cast<int64_t>(s) * stride + i];
    bad += (id < 0 || id >= num_blocks) ? 1 : 0;
  }
  if (bad) {
    atomicAdd(&result[0], bad);
    atomicMin(&result[1], s);
  }
}

// result = {0, INT32_MAX}: a kernel, not a memset, so the check may sit in a captured graph
__global__ void check_tables_reset_kernel(int32_t* result) {
  result[0] = 0;
  result[1] = 0x7FFFFFFF;
}

}  // namespace

hipError_t launch_check_tables(const int32_t* tables, int32_t stride, const int32_t* seq_lens, int32_t num_seqs,
                               int32_t block_size, int32_t num_blocks, int32_t max_seq_len, int32_t* result,
                               hipStream_t st) {
  check_tables_reset_kernel<<<1, 1, 0, st>>>(result);
  if (num_seqs > 0)
    check_tables_kernel<<<num_seqs, 256, 0, st>>>(tables, stride, seq_lens, block_size, num_blocks, max_seq_len,
                                                  result);
  return hipGetLastError();
}

hipError_t launch_move_blocks(const void* src_k, const void* src_v, int32_t src_blocks, void* dst_k, void* dst_v,
                              int32_t dst_blocks, const int32_t* pairs, int32_t n_pairs, int64_t block_bytes,
                              hipStream_t stream) {
  if (n_pairs == 0) return hipSuccess;
  // slices of at least 4 KiB per workgroup, at most 8 per block
  const int64_t slices = std::min<int64_t>(8, std::max<int64_t>(1, block_bytes / 4096));
  move_blocks_kernel<<<dim3(static_cast<unsigned>(n_pairs), 2, static_cast<unsigned>(slices)), dim3(256), 0,
                       stream>>>(src_k, src_v, dst_k, dst_v, pairs, src_blocks, dst_blocks, block_bytes);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n_pairs,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t stream) {
  return launch_move_blocks(k_pool, v_pool, num_blocks, k_pool, v_pool, num_blocks, pairs, n_pairs, block_bytes,
                            stream);
}

hipError_t launch_reshape_and_cache(const ScatterArgs& a, int dtype, hipStream_t stream) {
  const int esz = dtype == PKV_F32 ? 4 : 2;
  const int64_t work = 4 * static_cast<int64_t>(a.num_tokens) * a.n_kv_heads * (a.head_dim * esz / 16);  // threads
  if (work == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (work + threads - 1) / threads;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (esz == 4)
    reshape_and_cache_kernel<uint32_t><<<dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream>>>(a);
  else
    reshape_and_cache_kernel<uint16_t><<<dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const ScatterArgs& a, int src_dtype, float k_scale, float v_scale,
                                        hipStream_t stream) {
  const int64_t work = 4 * static_cast<int64_t>(a.num_tokens) * a.n_kv_heads * (a.head_dim / 16);  // threads
  if (work == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (work + threads - 1) / threads;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grd(static_cast<unsigned>(blocks)), blk(threads);
  if (src_dtype == PKV_F32) reshape_and_cache_fp8_kernel<float><<<grd, blk, 0, stream>>>(a, k_scale, v_scale);
  else if (src_dtype == PKV_F16) reshape_and_cache_fp8_kernel<_Float16><<<grd, blk, 0, stream>>>(a, k_scale, v_scale);
  else reshape_and_cache_fp8_kernel<__bf16><<<grd, blk, 0, stream>>>(a, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_append_slots(const int64_t* slot_mapping, int32_t num_seqs, int32_t* block_tables,
                               int32_t stride, int32_t* seq_lens, int32_t block_size,
                               hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  const int threads = 256;
  const int blocks = (num_seqs + threads - 1) / threads;
  append_slots_kernel<<<dim3(blocks), dim3(threads), 0, stream>>>(slot_mapping, num_seqs, block_tables,
                                                                  stride, seq_lens, block_size);
  return hipGetLastError();
}

}  // namespace pkv
