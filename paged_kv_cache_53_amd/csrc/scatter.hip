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
// reshape_and_cache_fp8 is the same scatter into a quantised cache: each
// element x is stored as the FP8 E4M3 code of x / scale (fp32 division,
// nearest code, ties to even, saturating at +-448, NaN to 0x7F), 16 codes per
// 16-byte key vector.
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

// FP8 E4M3 code of x: sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinities, S.1111.111
// is NaN, so the largest finite magnitude is 448.  Nearest code with ties to the even mantissa,
// magnitudes of 448 and above saturate to 448, NaN becomes 0x7F.
__device__ inline uint32_t e4m3_code(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;                 // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;         // |x| >= 448 (and infinities)
  if (a >= 0x3C800000u) {                            // |x| >= 2^-6: normal codes
    // keep 3 of the 23 mantissa bits, rounding to nearest even; a carry moves into the exponent.
    // Then rebias the exponent from 127 to 7: code = (e - 120) << 3 | m = (a' >> 20) - (120 << 3).
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((r >> 20) - (120u << 3));
  }
  // below 2^-6 the codes are the multiples of 2^-9 (code m = m * 2^-9, m <= 8 reaches the smallest
  // normal); |x| * 512 is exact and rintf rounds to nearest even
  return sign | static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
}

template <typename S> __device__ inline float src_f32(S x) { return static_cast<float>(x); }

// One thread: one 16-element key vector of one (token, head) and the 16 matching value elements.
template <typename S>  // source element type: float, _Float16 or __bf16
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(ScatterArgs a, float k_scale, float v_scale) {
  constexpr int X = 16;
  const int C = a.head_dim / X;
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
  const int64_t base = (blk * a.n_kv_heads + h) * static_cast<int64_t>(a.head_dim) * a.block_size;  // bytes

  constexpr int NV = X * sizeof(S) / 16;   // 16-byte source vectors per 16 elements
  const S* ksrc = static_cast<const S*>(a.k) + t * a.k_stride + static_cast<int64_t>(h) * a.head_dim + c * X;
  const S* vsrc = static_cast<const S*>(a.v) + t * a.v_stride + static_cast<int64_t>(h) * a.head_dim + c * X;
  uint4 kraw[NV], vraw[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    kraw[i] = reinterpret_cast<const uint4*>(ksrc)[i];
    vraw[i] = reinterpret_cast<const uint4*>(vsrc)[i];
  }
  S kx[X], vx[X];
  __builtin_memcpy(kx, kraw, sizeof(kx));
  __builtin_memcpy(vx, vraw, sizeof(vx));
  uint32_t kw[4] = {0u, 0u, 0u, 0u};
  uint8_t* kdst = static_cast<uint8_t*>(a.k_pool) + base + (static_cast<int64_t>(c) * a.block_size + off) * X;
  uint8_t* vdst = static_cast<uint8_t*>(a.v_pool) + base + static_cast<int64_t>(c) * X * a.block_size + off;
#pragma unroll
  for (int e = 0; e < X; ++e) {
    kw[e >> 2] |= e4m3_code(src_f32(kx[e]) / k_scale) << (8 * (e & 3));
    vdst[static_cast<int64_t>(e) * a.block_size] = static_cast<uint8_t>(e4m3_code(src_f32(vx[e]) / v_scale));
  }
  *reinterpret_cast<uint4*>(kdst) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
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

}  // namespace

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

hipError_t launch_reshape_and_cache_fp8(const ScatterArgs& a, int src_dtype, float k_scale, float v_scale,
                                        hipStream_t stream) {
  const int64_t work = static_cast<int64_t>(a.num_tokens) * a.n_kv_heads * (a.head_dim / 16);
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
