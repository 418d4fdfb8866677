// Slot-mapping scatter and the device half of the on-demand block append.
//
// reshape_and_cache writes every new token's key and value rows into the
// physical slot the block manager gave it ("PagedAttention -- Math + Memory
// Model", section "PagedAttention: blocks and the block table"); it copies
// bits, never converts.  One thread moves one 16-byte vector of a key row
// (X elements) and the X matching value elements:
//   key:   one 16-byte store to (blk, h, c, off, 0..X-1)   -- coalesced along c
//   value: X scalar stores to (blk, h, c*X + e, off)       -- the value pool keeps
//          tokens contiguous per head dimension for the decode kernel's PV reads
// append_slots records, per batch row, the block of the new token's slot in
// the row's block table and bumps the row's length.  copy_blocks makes the
// private copies of shared blocks that copy-on-write appends ask for.
#include <algorithm>

#include "pkv_internal.h"

namespace pkv {
namespace {

template <typename E>  // E: uint32_t (fp32) or uint16_t (fp16/bf16) -- raw bits
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ScatterArgs a) {
  constexpr int X = 16 / sizeof(E);
  const int C = a.head_dim / X;                       // 16-byte vectors per row
  const int64_t per_token = static_cast<int64_t>(a.n_kv_heads) * C;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= per_token * a.num_tokens) return;
  const int t = static_cast<int>(gid / per_token);
  const int rem = static_cast<int>(gid - static_cast<int64_t>(t) * per_token);
  const int h = rem / C;
  const int c = rem - h * C;
  const int64_t slot = a.slot_mapping[t];
  const int64_t cap = static_cast<int64_t>(a.num_blocks) * a.block_size;
  if (slot < 0 || slot >= cap) return;
  const int64_t blk = slot / a.block_size;
  const int off = static_cast<int>(slot - blk * a.block_size);
  const int64_t head_chunk = static_cast<int64_t>(a.head_dim) * a.block_size;  // elements
  const int64_t base = (blk * a.n_kv_heads + h) * head_chunk;

  const E* ksrc = static_cast<const E*>(a.k) + t * a.k_stride + static_cast<int64_t>(h) * a.head_dim + c * X;
  const E* vsrc = static_cast<const E*>(a.v) + t * a.v_stride + static_cast<int64_t>(h) * a.head_dim + c * X;
  const uint4 kv = *reinterpret_cast<const uint4*>(ksrc);
  const uint4 vv = *reinterpret_cast<const uint4*>(vsrc);

  E* kdst = static_cast<E*>(a.k_pool) + base + (static_cast<int64_t>(c) * a.block_size + off) * X;
  *reinterpret_cast<uint4*>(kdst) = kv;

  E vals[X];
  __builtin_memcpy(vals, &vv, 16);
  E* vdst = static_cast<E*>(a.v_pool) + base + static_cast<int64_t>(c) * X * a.block_size + off;
#pragma unroll
  for (int e = 0; e < X; ++e) vdst[static_cast<int64_t>(e) * a.block_size] = vals[e];
}

__global__ __launch_bounds__(256) void append_slots_kernel(const int64_t* __restrict__ slot_mapping,
                                                           int32_t num_seqs, int32_t* block_tables,
                                                           int32_t stride, int32_t* seq_lens,
                                                           int32_t block_size) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= num_seqs) return;
  const int64_t slot = slot_mapping[i];
  const int32_t p = seq_lens[i];
  if (slot < 0 || p < 0) return;
  const int32_t bi = p / block_size;
  if (bi >= stride) return;
  block_tables[static_cast<int64_t>(i) * stride + bi] = static_cast<int32_t>(slot / block_size);
  seq_lens[i] = p + 1;
}

// Copy-on-write: block dst of a pool becomes a copy of block src.  Grid: (pair, pool, slice);
// each workgroup moves one slice of one block with 16-byte loads and stores.
__global__ __launch_bounds__(256) void copy_blocks_kernel(void* k_pool, void* v_pool, const int32_t* pairs,
                                                          int32_t num_blocks, int64_t block_bytes) {
  const int src = pairs[2 * static_cast<int64_t>(blockIdx.x)];
  const int dst = pairs[2 * static_cast<int64_t>(blockIdx.x) + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks || src == dst) return;
  char* pool = static_cast<char*>(blockIdx.y ? v_pool : k_pool);
  const uint4* s = reinterpret_cast<const uint4*>(pool + src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>(pool + dst * block_bytes);
  const int64_t vecs = block_bytes / 16;
  for (int64_t i = static_cast<int64_t>(blockIdx.z) * blockDim.x + threadIdx.x; i < vecs;
       i += static_cast<int64_t>(gridDim.z) * blockDim.x)
    d[i] = s[i];
}

}  // namespace

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n_pairs,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t stream) {
  if (n_pairs == 0) return hipSuccess;
  // slices of at least 4 KiB per workgroup, at most 8 per block
  const int64_t slices = std::min<int64_t>(8, std::max<int64_t>(1, block_bytes / 4096));
  copy_blocks_kernel<<<dim3(static_cast<unsigned>(n_pairs), 2, static_cast<unsigned>(slices)), dim3(256), 0,
                       stream>>>(k_pool, v_pool, pairs, num_blocks, block_bytes);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const ScatterArgs& a, int dtype, hipStream_t stream) {
  const int esz = dtype == PKV_F32 ? 4 : 2;
  const int64_t work = static_cast<int64_t>(a.num_tokens) * a.n_kv_heads * (a.head_dim * esz / 16);
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
