// Per-thread bodies of the slot-mapping scatter, shared by the scatter kernels and the fused
// decode-step prologue (internal to libpagedkv).
//
// A 16-byte vector of one token's key row for one head (c-th vector of head h) and the matching
// value elements go into slot `slot` of the pools ("PagedAttention -- Math + Memory
// Model", section "PagedAttention: blocks and the block table": a new token goes to its slot in the
// block its table names):
//   key:   16 bytes to (blk, h, c, off, 0..X-1), four 4-byte stores by the four threads that share
//          the vector (one 16-byte segment)
//   value: X scalar stores to (blk, h, c*X + e, off), X/4 per thread -- the value pool keeps
//          tokens contiguous per head dimension for the decode kernel's value reads
// Slots outside the pools are skipped.  Item g of a scatter (thread 4g + sub) is vector
// c = g % C of head h = (g / C) % n_kv_heads of token t = g / (C * n_kv_heads), C = head_dim / X.
#pragma once

#include <type_traits>

#include "pkv_internal.h"

namespace pkv {

// Native pools: the rows' bits, unchanged.  E: uint32_t (fp32) or uint16_t (fp16/bf16).  Four threads share
// one key vector: thread `sub` (0..3) moves bytes 4*sub .. 4*sub+3 of it and the matching quarter of the
// value elements (X/4 of them), so a scatter spreads over four times as many threads.
template <typename E>
__device__ inline void scatter_quarter(const ScatterArgs& a, int t, int h, int c, int sub, int64_t slot) {
  constexpr int X = 16 / sizeof(E);
  constexpr int XQ = X / 4;   // value elements per quarter
  const int64_t cap = static_cast<int64_t>(a.num_blocks) * a.block_size;
  if (slot < 0 || slot >= cap) return;
  const int64_t blk = slot / a.block_size;
  const int off = static_cast<int>(slot - blk * a.block_size);
  const int64_t head_chunk = static_cast<int64_t>(a.head_dim) * a.block_size;  // elements
  const int64_t base = (blk * a.n_kv_heads + h) * head_chunk;

  const E* ksrc = static_cast<const E*>(a.k) + t * a.k_stride + static_cast<int64_t>(h) * a.head_dim + c * X;
  const E* vsrc = static_cast<const E*>(a.v) + t * a.v_stride + static_cast<int64_t>(h) * a.head_dim + c * X;
  const uint32_t kw = reinterpret_cast<const uint32_t*>(ksrc)[sub];
  const uint32_t vw = reinterpret_cast<const uint32_t*>(vsrc)[sub];

  E* kdst = static_cast<E*>(a.k_pool) + base + (static_cast<int64_t>(c) * a.block_size + off) * X;
  reinterpret_cast<uint32_t*>(kdst)[sub] = kw;

  E vals[XQ];
  __builtin_memcpy(vals, &vw, 4);
  E* vdst = static_cast<E*>(a.v_pool) + base + static_cast<int64_t>(c) * X * a.block_size + off;
#pragma unroll
  for (int e = 0; e < XQ; ++e) vdst[static_cast<int64_t>(sub * XQ + e) * a.block_size] = vals[e];
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

// FP8 pools: each element x is stored as the code of x / scale (IEEE fp32 division), 16 codes per 16-byte
// key vector.  S: the rows' element type (float, _Float16 or __bf16).  Four threads share one key vector:
// thread `sub` converts elements 4*sub .. 4*sub+3 of the key and of the value vector.
template <typename S>
__device__ inline void scatter_quarter_fp8(const ScatterArgs& a, int t, int h, int c, int sub, int64_t slot,
                                           float k_scale, float v_scale) {
  constexpr int X = 16;
  const int64_t cap = static_cast<int64_t>(a.num_blocks) * a.block_size;
  if (slot < 0 || slot >= cap) return;
  const int64_t blk = slot / a.block_size;
  const int off = static_cast<int>(slot - blk * a.block_size);
  const int64_t base = (blk * a.n_kv_heads + h) * static_cast<int64_t>(a.head_dim) * a.block_size;  // bytes

  using Raw = typename std::conditional<sizeof(S) == 4, uint4, uint2>::type;   // four source elements
  const S* ksrc = static_cast<const S*>(a.k) + t * a.k_stride + static_cast<int64_t>(h) * a.head_dim + c * X + 4 * sub;
  const S* vsrc = static_cast<const S*>(a.v) + t * a.v_stride + static_cast<int64_t>(h) * a.head_dim + c * X + 4 * sub;
  const Raw kraw = *reinterpret_cast<const Raw*>(ksrc);
  const Raw vraw = *reinterpret_cast<const Raw*>(vsrc);
  S kx[4], vx[4];
  __builtin_memcpy(kx, &kraw, sizeof(kx));
  __builtin_memcpy(vx, &vraw, sizeof(vx));
  uint32_t kw = 0u;
  uint8_t* kdst = static_cast<uint8_t*>(a.k_pool) + base + (static_cast<int64_t>(c) * a.block_size + off) * X;
  uint8_t* vdst = static_cast<uint8_t*>(a.v_pool) + base + static_cast<int64_t>(c) * X * a.block_size + off;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kw |= e4m3_code(static_cast<float>(kx[e]) / k_scale) << (8 * e);
    vdst[static_cast<int64_t>(4 * sub + e) * a.block_size] =
        static_cast<uint8_t>(e4m3_code(static_cast<float>(vx[e]) / v_scale));
  }
  reinterpret_cast<uint32_t*>(kdst)[sub] = kw;
}

// The device half of the on-demand append for batch row i: the block of the new token's slot goes
// into the row's table at the row's current length, and the length grows by one.  A negative slot
// or length, or a table already full, leaves the row unchanged.  Returns the row's length after.
__device__ inline int32_t append_row(const int64_t slot, int32_t* block_tables, int32_t stride, int32_t* seq_lens,
                                     int32_t block_size, int i) {
  const int32_t p = seq_lens[i];
  if (slot < 0 || p < 0) return p;
  const int32_t bi = p / block_size;
  if (bi >= stride) return p;
  block_tables[static_cast<int64_t>(i) * stride + bi] = static_cast<int32_t>(slot / block_size);
  seq_lens[i] = p + 1;
  return p + 1;
}

}  // namespace pkv
