// Paged decode attention for gfx950.
//
// What is computed: for each batch row s and query head h, softmax attention
// of q[s,h] over the row's L tokens, whose keys and values sit in the
// physical blocks its block table names ("PagedAttention -- Math + Memory
// Model", section "PagedAttention: blocks and the block table": the kernel
// reads the block table and gathers K and V from the scattered blocks for
// QK^T and the value-weighted sum; "KV-cache paging in vLLM", section "The
// Attention Kernel Change").
//
// How (MI355X design):
// * Work unit = (row, KV head, partition of part_tokens tokens).  A one-workgroup
//   plan kernel lists the (row, partition) pairs longest first, each with its row
//   length and first block id, so that opening a unit is one scalar load.  A
//   persistent grid of single-wave workgroups takes the list's first rounds in a
//   fixed order (round r: one unit per wave) and the rest from one atomic counter,
//   so no wave is launched for a partition that does not exist and long and short
//   rows balance across the 256 CUs.
// * A wave streams its units in tiles (16 tokens; 32 for an FP8 cache) through NB
//   register buffers, NB - 1 tiles in flight: while tile t is computed, tiles
//   t+1 .. t+NB-1 are loading.  Streamed batches run one wave per SIMD with five
//   buffers (FP8: four); batches whose rows share blocks run two waves per SIMD
//   with three.  The issue side runs ahead across unit boundaries (it opens the
//   next unit a few tiles before the current one ends and loads that unit's q
//   straight into LDS), so HBM sees no gap between units.  When nothing real is
//   left to issue it issues filler loads of an already-loaded tile, which keeps
//   the number of loads per step fixed: the wait before a tile's use then covers
//   that tile only.
// * Block ids, lengths and the unit list are read with scalar loads, which wait
//   on their own counter and never stall behind the vector loads.
// * Key rows are stored as 16-byte vectors [c][token][X]: the 64 lanes of a
//   wave read 1 KiB contiguous per load (lane = token within 16, lane group =
//   vector column).  Values are stored [dim][token] so that a lane's 4
//   consecutive tokens of one dimension are one 8-byte load -- exactly the
//   operand the PV product contracts over.
// * MFMA path (16-bit KV, any G <= 16): S^T = K q^T and O^T = V^T P^T with
//   v_mfma_f32_16x16x32_{bf16,f16} and v_mfma_f32_16x16x16{bf16_1k,f16}; the G
//   query heads of a KV head are the 16-wide N dimension (padded).  The QK
//   accumulator layout (lane holds tokens 4g..4g+3 for head lane%16) is exactly
//   the B operand layout of the PV product, so weights never leave their lanes.
//   The weights are rounded to the KV type for the PV operand, and the
//   denominator sums the rounded values.
// * Quantised KV (FP8 E4M3 codes with per-tensor scales, q and output in bf16
//   or f16): the same MFMA products after widening the codes in registers to
//   q's type, which holds every E4M3 value exactly.  A key vector is 16 codes
//   (16 bytes), so a lane's q fragments take the matching dims; the key scale
//   is folded into the score scale and the value scale into the output.  Its
//   tiles hold 32 tokens, so that a tile has the bytes and the load widths of
//   a 16-bit one (the QK rows are ordered so that the scores land in the
//   operand layout of a 32-deep PV MFMA).
// * Vector path (fp32 KV, and 16-bit KV with one query head per KV head on
//   request): per-token dot products with a 4-lane cross-group reduction, fp32
//   weights, FMA accumulation.
// * Loads: streamed with the non-temporal hint by default; cacheable for a batch
//   whose rows share blocks; or chosen per tile (cacheable inside the rows'
//   shared prefix, streamed after it) by one scalar branch inside each group
//   of loads, which keeps a single load sequence for the waits.
// * q fragments live in LDS (one slot for the unit being computed, one for the
//   unit being issued), so the tile buffers keep the registers.
// * Online softmax in the base-2 domain (scores pre-multiplied by
//   scale*log2(e), v_exp_f32); the accumulators are rescaled only on tiles
//   where some lane's running max rose (elsewhere the factor is exactly 1);
//   masked tokens get -inf scores and zeroed value elements (selected, never
//   multiplied, so a NaN in an unused slot cannot leak in).  Rows with one partition write the output directly; longer rows
//   write (max, sum, acc) partials that the reduce kernel merges.
#include <type_traits>
#include <utility>

#include "pkv_internal.h"
#include "scatter_body.h"

namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> { using type = bf16x8; };
template <> struct Vec8<_Float16> { using type = f16x8; };

__device__ inline f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of `v` in lane `src` (0..63) of the wave.
__device__ inline int lane_fetch(int v, int src) { return __builtin_amdgcn_ds_bpermute(src << 2, v); }
__device__ inline float lane_fetch(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

__device__ inline float xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Symmetric reductions with lane ^ 16 and lane ^ 32 through the gfx950 row and half swaps
// (v_permlane16_swap / v_permlane32_swap), which exchange inside the VALU instead of through LDS as a
// shuffle does.  With both operands equal, each lane gets its own value and its partner's, in an
// order that depends on the lane; a maximum or a sum of the two is the same either way (IEEE
// addition is commutative, so sums are bit-identical to the shuffle form).
__device__ inline float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T> __device__ inline float to_f32(T x) { return static_cast<float>(x); }

// Finished results (outputs and partials) are written through to memory (the sc1 policy).  A
// store stays in the wave's vector-memory queue until acknowledged, and the loads issued after
// it cannot retire before it; write-through stores measured 4 % faster on the long workloads
// than write-back ones.  The cache policy needs inline assembly; the nop after a 16-byte store
// covers the hazard of a following VALU write to the stored registers, which the compiler
// cannot see through the asm.  Nothing in the decode kernel reads what these stores write.
__device__ inline void st_wt(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" :: "v"(p), "v"(v));
}
__device__ inline void st_wt(void* p, u32x2 v) {
  asm volatile("global_store_dwordx2 %0, %1, off sc1" :: "v"(p), "v"(v));
}
__device__ inline void st_wt(float* p, float v) {
  asm volatile("global_store_dword %0, %1, off sc1" :: "v"(p), "v"(v));
}
__device__ inline void st_wt16(void* p, unsigned bits) {
  asm volatile("global_store_short %0, %1, off sc1" :: "v"(p), "v"(bits));
}

// Stores 4 consecutive output elements (16-bit KV types, or fp32 output).
template <typename T>
__device__ inline void store4(void* out, int64_t idx, f32x4 v, bool f32out) {
  if (f32out) {
    st_wt(static_cast<float*>(out) + idx, v);
  } else {
    static_assert(sizeof(T) == 2, "4 elements of a 16-bit type");
    T t[4] = {static_cast<T>(v[0]), static_cast<T>(v[1]), static_cast<T>(v[2]), static_cast<T>(v[3])};
    u32x2 bits;
    __builtin_memcpy(&bits, t, 8);
    st_wt(static_cast<T*>(out) + idx, bits);
  }
}
template <typename T>
__device__ inline void store1(void* out, int64_t idx, float v, bool f32out) {
  if (f32out || sizeof(T) == 4) {
    st_wt(static_cast<float*>(out) + idx, v);
  } else {
    const T t = static_cast<T>(v);
    unsigned short b;
    __builtin_memcpy(&b, &t, 2);
    st_wt16(static_cast<T*>(out) + idx, b);
  }
}

// Wave-uniform read of memory no kernel of this launch writes (lengths, block table, unit list):
// the constant address space lets the compiler use scalar loads, which wait on lgkmcnt and so
// never make a wave wait for its outstanding vector loads.
__device__ inline int ld_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)(p))[i];
}

__device__ inline int row_len(const DecodeArgs& a, int s) {
  const int L = ld_uniform(a.seq_lens, s);
  return L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
}

// ------------------------------------------------------------------------------ plan
// Inclusive prefix sum of v over the 1024 threads of a workgroup: a shuffle scan inside each
// 64-lane wave, one wave scanning the 16 wave totals, then each wave adds its predecessors' total.
// *total receives the sum over all threads.  wave_sums: 16 ints of LDS.
__device__ inline int block_scan_1024(int v, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    v += lane >= d ? t : 0;
  }
  __syncthreads();   // wave_sums may still be read by a previous scan
  if (lane == 63) wave_sums[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? wave_sums[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int t = __shfl_up(w, d, 64);
      w += lane >= d ? t : 0;
    }
    if (lane < 16) wave_sums[lane] = w;
  }
  __syncthreads();
  *total = wave_sums[15];
  return v + (wave > 0 ? wave_sums[wave - 1] : 0);
}

// Lists the (row, partition) pairs, largest first: every full partition, then each row's
// shorter last partition in decreasing length (counting sort over 16-token buckets).  Waves
// claim units in this order, so the last units handed out are the shortest and the waves
// finish together.  The order decides only which wave computes a unit, never its result.
// Run by one workgroup of 1024 threads; thread t reads the lengths of rows t*per .. t*per+per-1
// only (len_of(s): row s's length, clamped to 0 .. max_seq_len), in two passes.
template <typename T, class LenOf>
__device__ inline void plan_units(const DecodeArgs& a, int head_dim, LenOf len_of) {
  constexpr int NBUCKET = 1024;
  __shared__ int wave_sums[16];
  __shared__ int bucket_base[NBUCKET];
  __shared__ int bucket_fill[NBUCKET];
  const int S = a.num_seqs;
  const int P = a.part_tokens;
  const int tid = threadIdx.x;
  int shift = 4;
  while (((P - 1) >> shift) >= NBUCKET) ++shift;
  const int per = (S + 1023) / 1024;
  const int lo = min(S, tid * per);
  const int hi = min(S, lo + per);
  for (int i = tid; i < NBUCKET; i += 1024) bucket_fill[i] = 0;
  __syncthreads();
  int full_local = 0;
  for (int s = lo; s < hi; ++s) {
    const int L = len_of(s);
    full_local += L / P;
    if (L % P) atomicAdd(&bucket_fill[((L % P) - 1) >> shift], 1);
  }
  int full_total = 0;
  int off = block_scan_1024(full_local, wave_sums, &full_total) - full_local;   // (its barriers order the counts)
  // bucket bases, longest bucket first, after all full partitions: an exclusive scan of the
  // bucket counts taken in descending bucket order (thread t holds bucket NBUCKET-1-t)
  const int rb = NBUCKET - 1 - tid;
  const int cnt = bucket_fill[rb];
  int part_total = 0;
  const int incl = block_scan_1024(cnt, wave_sums, &part_total);
  bucket_base[rb] = full_total + incl - cnt;
  bucket_fill[rb] = 0;
  if (tid == 0) a.counters[0] = full_total + part_total;
  if (tid == 1) a.counters[17] = full_total;
  __syncthreads();
  const int64_t row_elems = static_cast<int64_t>(a.n_q_heads) * head_dim;
  for (int s = lo; s < hi; ++s) {
    const int L = len_of(s);
    const int nfull = L / P;
    for (int p = 0; p < nfull; ++p) a.units[off + p] = make_int4(s, p, L, 0);
    off += nfull;
    if (L % P) {
      const int bk = ((L % P) - 1) >> shift;
      a.units[bucket_base[bk] + atomicAdd(&bucket_fill[bk], 1)] = make_int4(s, nfull, L, 0);
    }
    if (L == 0) {  // empty row: zeros
      for (int64_t i = 0; i < row_elems; ++i) store1<T>(a.out, s * row_elems + i, 0.f, a.out_f32);
    }
  }
  if (tid >= 1 && tid <= 16) a.counters[tid] = 0;   // work-claim counters
  // Second pass, one pair per thread at a time: the block id of each partition's first block, so that
  // opening a unit is one scalar load.  (The workgroup barrier makes the first pass's stores visible.)
  __syncthreads();
  const int npairs = full_total + part_total;
  for (int i = tid; i < npairs; i += 1024) {
    const int4 u = a.units[i];
    const int blk = (u.y * P) >> a.log2_block;
    a.units[i].w = a.flat_bps > 0 ? a.block_tables[u.x] * a.flat_bps + blk
                                  : a.block_tables[static_cast<int64_t>(u.x) * a.bt_stride + blk];
  }
}

template <typename T>
__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a, int head_dim) {
  plan_units<T>(a, head_dim, [&](int s) { return row_len(a, s); });
}

// ------------------------------------------------------------------------------ fused step prologue
// The first kernel of a fused decode step: the device append, the scatter of the new tokens and the
// plan, in one launch.  Workgroup 0 appends each row's new token (its block into the row's table,
// the length up by one) and then plans over the lengths it has just written: each of its threads
// appends and later reads back the same rows, so its own ordinary loads see its own stores.  The
// other workgroups scatter the new tokens' keys and values, 256 key vectors per workgroup and four
// threads per vector, after staging their tokens' slots in LDS (the slot mapping may live in pinned
// host memory, so each slot is read once per workgroup that needs it).  The scatter and the append touch disjoint memory
// and the plan reads only lengths, so the parts need no ordering between workgroups.
template <typename T, bool FP8>
__global__ __launch_bounds__(1024) void step_prologue_kernel(DecodeArgs a, ScatterArgs sc, StepArgs st,
                                                             int head_dim) {
  if (blockIdx.x == 0) {
    const int S = a.num_seqs;
    const int per = (S + 1023) / 1024;
    const int lo = min(S, static_cast<int>(threadIdx.x) * per);
    const int hi = min(S, lo + per);
    for (int s = lo; s < hi; ++s) append_row(st.slots[s], st.block_tables, a.bt_stride, st.seq_lens, a.block_size, s);
    plan_units<T>(a, head_dim, [&](int s) {
      const int L = st.seq_lens[s];
      return L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
    });
    return;
  }
  constexpr int C_ELEM = FP8 ? 16 : 16 / static_cast<int>(sizeof(T));   // elements per key vector
  constexpr int kItems = 1024 / 4;           // key vectors per workgroup, four threads each
  constexpr int kMaxTok = kItems / 4 + 2;    // 4 or more vectors per token (head_dim >= 64)
  __shared__ int64_t slot_lds[kMaxTok];
  const int C = sc.head_dim / C_ELEM;
  const int64_t per_token = static_cast<int64_t>(sc.n_kv_heads) * C;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x - 1) * kItems;   // this workgroup's first vector
  const int64_t total = per_token * sc.num_tokens;
  const int t_first = static_cast<int>(i0 / per_token);
  const int t_end = static_cast<int>(min(total - 1, i0 + kItems - 1) / per_token) + 1;   // past the last token
  if (static_cast<int>(threadIdx.x) < min(t_end - t_first, kMaxTok))
    slot_lds[threadIdx.x] = st.slots[t_first + threadIdx.x];
  __syncthreads();
  const int64_t item = i0 + (threadIdx.x >> 2);
  if (item >= total) return;
  const int sub = threadIdx.x & 3;
  const int t = static_cast<int>(item / per_token);
  const int rem = static_cast<int>(item - static_cast<int64_t>(t) * per_token);
  const int h = rem / C;
  const int c = rem - h * C;
  if (t - t_first >= kMaxTok) return;   // (the host admits head_dim >= 64 only)
  const int64_t slot = slot_lds[t - t_first];
  if constexpr (FP8) {
    scatter_quarter_fp8<T>(sc, t, h, c, sub, slot, st.k_scale, st.v_scale);
  } else {
    using E = typename std::conditional<sizeof(T) == 4, uint32_t, uint16_t>::type;
    scatter_quarter<E>(sc, t, h, c, sub, slot);
  }
}

// ------------------------------------------------------------------------------ tile pipeline
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Explicitly waited vector-memory operations.  The tile stream's loads, the early q loads and
// the work-claim atomic are issued through inline assembly, which the compiler's wait
// insertion does not track; across the pipeline's branches its merged bookkeeping otherwise
// drains every outstanding load before each new tile is issued.  Each operation names its
// destination as an in/out operand, so those registers stay with their buffer for the whole
// loop and are never reused as temporaries, and every use of the loaded data comes after an
// explicit "s_waitcnt vmcnt(N)" followed by tie() on the same registers, where N is a count of
// vector-memory instructions the pipeline always issues after the operation.  vmcnt counts
// loads, stores and atomics together and they retire in order, so waiting for at most N
// outstanding, with N no larger than the number issued since, guarantees completion.
// Tile loads carry the non-temporal hint by default: the key and value stream is read once per
// call, and keeping it from displacing other lines in L2 and the Infinity Cache measured 5 %
// faster (the partial results the merge kernel reads next stay resident).
// With E false (tiles too large to keep three in registers without spilling, where a spill of
// an in-flight register would be wrong) every helper is the ordinary compiler-tracked form.
// NT selects the non-temporal hint (the caller's choice: off when blocks are shared by rows of
// the batch and are worth keeping in cache).
template <bool E, bool NT>
__device__ inline void vload(u32x4& d, const void* p) {
  if constexpr (E && NT) asm volatile("global_load_dwordx4 %0, %1, off nt" : "+v"(d) : "v"(p));
  else if constexpr (E) asm volatile("global_load_dwordx4 %0, %1, off" : "+v"(d) : "v"(p));
  else if constexpr (NT) d = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  else d = *static_cast<const u32x4*>(p);
}
template <bool E, bool NT>
__device__ inline void vload(u32x2& d, const void* p) {
  if constexpr (E && NT) asm volatile("global_load_dwordx2 %0, %1, off nt" : "+v"(d) : "v"(p));
  else if constexpr (E) asm volatile("global_load_dwordx2 %0, %1, off" : "+v"(d) : "v"(p));
  else if constexpr (NT) d = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
  else d = *static_cast<const u32x2*>(p);
}
template <bool E, bool NT>
__device__ inline void vload(unsigned& d, const void* p) {
  if constexpr (E && NT) asm volatile("global_load_dword %0, %1, off nt" : "+v"(d) : "v"(p));
  else if constexpr (E) asm volatile("global_load_dword %0, %1, off" : "+v"(d) : "v"(p));
  else if constexpr (NT) d = __builtin_nontemporal_load(static_cast<const unsigned*>(p));
  else d = *static_cast<const unsigned*>(p);
}
// The loads of a tile at constant byte strides from one address: the strides go into the
// instructions' immediate offsets (at most 4095 bytes), so the group needs one address register pair
// instead of one per load.  Larger strides keep one address per load.
template <bool E, bool NT, int OFF>
__device__ inline void vload_at(u32x4& d, const void* p) {
  if constexpr (E && NT) asm volatile("global_load_dwordx4 %0, %1, off offset:%2 nt" : "+v"(d) : "v"(p), "i"(OFF));
  else if constexpr (E) asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "+v"(d) : "v"(p), "i"(OFF));
  else vload<E, NT>(d, static_cast<const char*>(p) + OFF);
}
template <bool E, bool NT, int OFF>
__device__ inline void vload_at(u32x2& d, const void* p) {
  if constexpr (E && NT) asm volatile("global_load_dwordx2 %0, %1, off offset:%2 nt" : "+v"(d) : "v"(p), "i"(OFF));
  else if constexpr (E) asm volatile("global_load_dwordx2 %0, %1, off offset:%2" : "+v"(d) : "v"(p), "i"(OFF));
  else vload<E, NT>(d, static_cast<const char*>(p) + OFF);
}
template <bool E, bool NT, int STRIDE, typename Dst, size_t... I>
__device__ inline void vload_strided_seq(Dst* d, const void* p, std::index_sequence<I...>) {
  if constexpr ((sizeof...(I) - 1) * STRIDE <= 4095) {
    (vload_at<E, NT, static_cast<int>(I) * STRIDE>(d[I], p), ...);
  } else {
    (vload<E, NT>(d[I], static_cast<const char*>(p) + static_cast<int>(I) * STRIDE), ...);
  }
}
template <bool E, bool NT, int STRIDE, int N, typename Dst>
__device__ inline void vload_strided(Dst (&d)[N], const void* p) {
  vload_strided_seq<E, NT, STRIDE>(d, p, std::make_index_sequence<N>{});
}

// Per-tile choice of the load policy: a group of loads issued in one asm statement whose one scalar
// branch picks the cacheable or the non-temporal form of every load (cached: wave-uniform, nonzero for
// cacheable).  Both paths issue the same loads into the same registers, so the statement counts the
// same on vmcnt either way, and the compiler sees a single definition of each register: two separate
// load sequences under a branch of its own meet in a merge that it may resolve by copying the loaded
// registers before the data arrives.  (Explicitly waited kernels only.)
__device__ inline void vload_sel(u32x4& d0, u32x4& d1, const void* p0, const void* p1, unsigned cached) {
  const unsigned c = __builtin_amdgcn_readfirstlane(cached);   // (a scalar operand)
  asm volatile(
      "s_cmp_eq_u32 %4, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "global_load_dwordx4 %0, %2, off\n\t"
      "global_load_dwordx4 %1, %3, off\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "global_load_dwordx4 %0, %2, off nt\n\t"
      "global_load_dwordx4 %1, %3, off nt\n"
      "2:"
      : "+v"(d0), "+v"(d1)
      : "v"(p0), "v"(p1), "s"(c)
      : "scc");
}
__device__ inline void vload_sel(u32x4& d0, u32x4& d1, u32x4& d2, u32x4& d3, const void* p0, const void* p1, const void* p2, const void* p3, unsigned cached) {
  const unsigned c = __builtin_amdgcn_readfirstlane(cached);   // (a scalar operand)
  asm volatile(
      "s_cmp_eq_u32 %8, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "global_load_dwordx4 %0, %4, off\n\t"
      "global_load_dwordx4 %1, %5, off\n\t"
      "global_load_dwordx4 %2, %6, off\n\t"
      "global_load_dwordx4 %3, %7, off\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "global_load_dwordx4 %0, %4, off nt\n\t"
      "global_load_dwordx4 %1, %5, off nt\n\t"
      "global_load_dwordx4 %2, %6, off nt\n\t"
      "global_load_dwordx4 %3, %7, off nt\n"
      "2:"
      : "+v"(d0), "+v"(d1), "+v"(d2), "+v"(d3)
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3), "s"(c)
      : "scc");
}
__device__ inline void vload_sel(u32x2& d0, u32x2& d1, u32x2& d2, u32x2& d3, const void* p0, const void* p1, const void* p2, const void* p3, unsigned cached) {
  const unsigned c = __builtin_amdgcn_readfirstlane(cached);   // (a scalar operand)
  asm volatile(
      "s_cmp_eq_u32 %8, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "global_load_dwordx2 %0, %4, off\n\t"
      "global_load_dwordx2 %1, %5, off\n\t"
      "global_load_dwordx2 %2, %6, off\n\t"
      "global_load_dwordx2 %3, %7, off\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "global_load_dwordx2 %0, %4, off nt\n\t"
      "global_load_dwordx2 %1, %5, off nt\n\t"
      "global_load_dwordx2 %2, %6, off nt\n\t"
      "global_load_dwordx2 %3, %7, off nt\n"
      "2:"
      : "+v"(d0), "+v"(d1), "+v"(d2), "+v"(d3)
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3), "s"(c)
      : "scc");
}
__device__ inline void vload_sel(u32x2& d0, u32x2& d1, u32x2& d2, u32x2& d3, u32x2& d4, u32x2& d5, u32x2& d6, u32x2& d7, const void* p0, const void* p1, const void* p2, const void* p3, const void* p4, const void* p5, const void* p6, const void* p7, unsigned cached) {
  const unsigned c = __builtin_amdgcn_readfirstlane(cached);   // (a scalar operand)
  asm volatile(
      "s_cmp_eq_u32 %16, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "global_load_dwordx2 %0, %8, off\n\t"
      "global_load_dwordx2 %1, %9, off\n\t"
      "global_load_dwordx2 %2, %10, off\n\t"
      "global_load_dwordx2 %3, %11, off\n\t"
      "global_load_dwordx2 %4, %12, off\n\t"
      "global_load_dwordx2 %5, %13, off\n\t"
      "global_load_dwordx2 %6, %14, off\n\t"
      "global_load_dwordx2 %7, %15, off\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "global_load_dwordx2 %0, %8, off nt\n\t"
      "global_load_dwordx2 %1, %9, off nt\n\t"
      "global_load_dwordx2 %2, %10, off nt\n\t"
      "global_load_dwordx2 %3, %11, off nt\n\t"
      "global_load_dwordx2 %4, %12, off nt\n\t"
      "global_load_dwordx2 %5, %13, off nt\n\t"
      "global_load_dwordx2 %6, %14, off nt\n\t"
      "global_load_dwordx2 %7, %15, off nt\n"
      "2:"
      : "+v"(d0), "+v"(d1), "+v"(d2), "+v"(d3), "+v"(d4), "+v"(d5), "+v"(d6), "+v"(d7)
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3), "v"(p4), "v"(p5), "v"(p6), "v"(p7), "s"(c)
      : "scc");
}
template <int N> __device__ inline void vload_group(u32x4 (&d)[N], const void* const (&p)[N], unsigned c) {
  static_assert(N == 2 || N == 4, "groups of 2 or 4 16-byte loads");
  if constexpr (N == 2) vload_sel(d[0], d[1], p[0], p[1], c);
  else vload_sel(d[0], d[1], d[2], d[3], p[0], p[1], p[2], p[3], c);
}
template <int N> __device__ inline void vload_group(u32x2 (&d)[N], const void* const (&p)[N], unsigned c) {
  static_assert(N == 4 || N == 8, "groups of 4 or 8 8-byte loads");
  if constexpr (N == 4) vload_sel(d[0], d[1], d[2], d[3], p[0], p[1], p[2], p[3], c);
  else vload_sel(d[0], d[1], d[2], d[3], d[4], d[5], d[6], d[7], p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], c);
}

// vload_group for loads at constant byte strides from one address (immediate offsets, at most 4095
// bytes): one address register pair for the whole group.
template <int S>
__device__ inline void vload_sel_strided(u32x4 (&d)[2], const void* p, unsigned cached) {
  const unsigned c = __builtin_amdgcn_readfirstlane(cached);   // (a scalar operand)
  asm volatile(
      "s_cmp_eq_u32 %3, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "global_load_dwordx4 %0, %2, off\n\t"
      "global_load_dwordx4 %1, %2, off offset:%4\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "global_load_dwordx4 %0, %2, off nt\n\t"
      "global_load_dwordx4 %1, %2, off offset:%4 nt\n"
      "2:"
      : "+v"(d[0]), "+v"(d[1])
      : "v"(p), "s"(c), "i"(S)
      : "scc");
}
template <int S>
__device__ inline void vload_sel_strided(u32x4 (&d)[4], const void* p, unsigned cached) {
  const unsigned c = __builtin_amdgcn_readfirstlane(cached);   // (a scalar operand)
  asm volatile(
      "s_cmp_eq_u32 %5, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "global_load_dwordx4 %0, %4, off\n\t"
      "global_load_dwordx4 %1, %4, off offset:%6\n\t"
      "global_load_dwordx4 %2, %4, off offset:%7\n\t"
      "global_load_dwordx4 %3, %4, off offset:%8\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "global_load_dwordx4 %0, %4, off nt\n\t"
      "global_load_dwordx4 %1, %4, off offset:%6 nt\n\t"
      "global_load_dwordx4 %2, %4, off offset:%7 nt\n\t"
      "global_load_dwordx4 %3, %4, off offset:%8 nt\n"
      "2:"
      : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3])
      : "v"(p), "s"(c), "i"(S), "i"(2 * S), "i"(3 * S)
      : "scc");
}
template <int S>
__device__ inline void vload_sel_strided(u32x2 (&d)[8], const void* p, unsigned cached) {
  const unsigned c = __builtin_amdgcn_readfirstlane(cached);   // (a scalar operand)
  asm volatile(
      "s_cmp_eq_u32 %9, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "global_load_dwordx2 %0, %8, off\n\t"
      "global_load_dwordx2 %1, %8, off offset:%10\n\t"
      "global_load_dwordx2 %2, %8, off offset:%11\n\t"
      "global_load_dwordx2 %3, %8, off offset:%12\n\t"
      "global_load_dwordx2 %4, %8, off offset:%13\n\t"
      "global_load_dwordx2 %5, %8, off offset:%14\n\t"
      "global_load_dwordx2 %6, %8, off offset:%15\n\t"
      "global_load_dwordx2 %7, %8, off offset:%16\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "global_load_dwordx2 %0, %8, off nt\n\t"
      "global_load_dwordx2 %1, %8, off offset:%10 nt\n\t"
      "global_load_dwordx2 %2, %8, off offset:%11 nt\n\t"
      "global_load_dwordx2 %3, %8, off offset:%12 nt\n\t"
      "global_load_dwordx2 %4, %8, off offset:%13 nt\n\t"
      "global_load_dwordx2 %5, %8, off offset:%14 nt\n\t"
      "global_load_dwordx2 %6, %8, off offset:%15 nt\n\t"
      "global_load_dwordx2 %7, %8, off offset:%16 nt\n"
      "2:"
      : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]), "+v"(d[4]), "+v"(d[5]), "+v"(d[6]), "+v"(d[7])
      : "v"(p), "s"(c), "i"(S), "i"(2 * S), "i"(3 * S), "i"(4 * S), "i"(5 * S), "i"(6 * S), "i"(7 * S)
      : "scc");
}
// the strided group where its offsets fit the instructions, else one address per load
template <int S, int N, typename Dst>
__device__ inline void vload_group_strided(Dst (&d)[N], const void* p, unsigned cached) {
  if constexpr ((N - 1) * S <= 4095 && (N == 2 || N == 4 || N == 8) &&
                (std::is_same<Dst, u32x4>::value ? N != 8 : N == 8)) {
    vload_sel_strided<S>(d, p, cached);
  } else {
    const void* a[N];
#pragma unroll
    for (int i = 0; i < N; ++i) a[i] = static_cast<const char*>(p) + i * S;
    vload_group(d, a, cached);
  }
}

// waits until at most N vector-memory operations are outstanding
// (the memory clobber keeps every memory access of the source on its side of the wait: a read of
// LDS that a global-to-LDS load fills must not be scheduled above the wait that retires that load)
template <bool E, int N> __device__ inline void vm_wait() {
  static_assert(!E || (N >= 0 && N < 64), "vmcnt holds 6 bits");
  if constexpr (E) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// orders every later use of r after the preceding wait
template <bool E, typename R> __device__ inline void tie(R& r) { if constexpr (E) asm volatile("" : "+v"(r)); }

// Storage element of a quantised cache: one FP8 E4M3 code.
struct E4M3 {
  unsigned char bits;
};

// Storage traits: X elements per 16-byte key vector; VV holds 4 consecutive tokens of one
// value dimension.
template <typename T> struct Kv;
template <> struct Kv<__bf16> { static constexpr int X = 8; using VV = u32x2; };
template <> struct Kv<_Float16> { static constexpr int X = 8; using VV = u32x2; };
template <> struct Kv<float> { static constexpr int X = 4; using VV = u32x4; };
template <> struct Kv<E4M3> { static constexpr int X = 16; using VV = unsigned; };

// One work unit (row s, KV head kvh, partition part); all fields are wave-uniform.
template <typename T>
struct Unit {
  int s, kvh, part, ntok, nparts;
  int id_first;       // the partition's first block id, read when the unit is opened
  const int32_t* bt;  // block-table row at the partition's first block
};

// FLAT: the row's blocks are the consecutive blocks of its span (block_tables holds one span index
// per row): the first block id is computed, not read from a table.
// One scalar load of the unit's descriptor {row, partition, row length, first block id}, which the
// plan wrote (FLAT: the first block id follows from the row's span, no table is read).
template <typename T, bool FLAT>
__device__ inline Unit<T> open_unit(const DecodeArgs& a, int id, int64_t chunk) {
  Unit<T> u;
  const int pair = id / a.n_kv_heads;
  u.kvh = id - pair * a.n_kv_heads;
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 d = ((const __attribute__((address_space(4))) i32x4*)(a.units))[pair];
  u.s = d.x;
  u.part = d.y;
  const int L = d.z;
  const int tok0 = u.part * a.part_tokens;
  u.ntok = min(a.part_tokens, L - tok0);
  u.nparts = (L + a.part_tokens - 1) / a.part_tokens;
  u.id_first = d.w;
  if constexpr (FLAT) {
    u.bt = a.block_tables;   // unused
  } else {
    u.bt = a.block_tables + static_cast<int64_t>(u.s) * a.bt_stride + (tok0 >> a.log2_block);
  }
  (void)chunk;
  return u;
}

// Register-resident tile of 16 tokens.  Keys: lane (token lane%16, group g = lane/16) holds
// the 16-byte vectors 4ks+g of its token's row (the A operand of the MFMA QK product, and the
// vector path's share of the dot product).  Values: lane (dim 16dt + lane%16, group g) holds
// tokens 4g..4g+3 of that dim (the A operand of the MFMA PV product).
template <typename T, int D>
struct Tile16 {
  static constexpr int kTokens = 16;
  static constexpr int NK = D / Kv<T>::X / 4;
  static constexpr int kLoads = NK + D / 16;   // vector-memory instructions per tile
  u32x4 kf[NK];
  typename Kv<T>::VV vf[D / 16];

  // Issues the kLoads loads of the tile at partition offset t0 of a unit (block table row bt,
  // ntok tokens, pools offset to its KV head), completion explicitly waited when E (vload).
  // Block ids are wave-uniform scalar loads (the first one was read when the unit was opened);
  // table entries past the unit's last block are never read (those tokens reuse the first id
  // and are masked in the compute).  FLAT: block i of the unit is id_first + i, no table.
  template <int Bsz, bool E, bool NT, bool FLAT, bool MIX = false>
  __device__ void issue(const DecodeArgs& a, const int32_t* bt, int id_first, int ntok, const T* kbase,
                        const T* vbase, int t0, int64_t blk_stride, unsigned cached = 0) {
    constexpr int X = Kv<T>::X;
    constexpr int NB = Bsz >= 16 ? 1 : 16 / Bsz;   // blocks per tile
    const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
    const int first = t0 / Bsz;
    int id0 = FLAT ? id_first + first : (first == 0 ? id_first : ld_uniform(bt, first));
    int id1 = id0;
    if constexpr (NB == 2) {
      if (t0 + 8 < ntok) id1 = FLAT ? id_first + first + 1 : ld_uniform(bt, first + 1);
    }
    id0 = min(max(id0, 0), a.num_blocks - 1);
    id1 = min(max(id1, 0), a.num_blocks - 1);
    const int bk = (NB == 2 && r16 >= 8) ? id1 : id0;
    const T* kb = kbase + static_cast<int64_t>(bk) * blk_stride + (((t0 + r16) & (Bsz - 1)) + g * Bsz) * X;
    if constexpr (MIX) {
      vload_group_strided<4 * Bsz * X * static_cast<int>(sizeof(T))>(kf, kb, cached);
    } else {
      vload_strided<E, NT, 4 * Bsz * X * static_cast<int>(sizeof(T))>(kf, kb);
    }
    const int bv = (NB == 2 && g >= 2) ? id1 : id0;
    const T* vb = vbase + static_cast<int64_t>(bv) * blk_stride + r16 * Bsz + ((t0 + 4 * g) & (Bsz - 1));
    // A block of more than 16 tokens holds each value dim's tokens in a row longer than the tile's
    // share: the tile reads half of every line and the next tile the other half, so those lines
    // stay cacheable (the non-temporal hint made the second half come from HBM again: 1115 us
    // instead of 840 us on the Llama-70B-class batch at B = 32).  Key lines are read whole.
    constexpr bool kNTV = NT && Bsz <= 16;
    if constexpr (MIX) {
      vload_group_strided<16 * Bsz * static_cast<int>(sizeof(T))>(vf, vb, Bsz <= 16 ? cached : 1u);
    } else {
      vload_strided<E, kNTV, 16 * Bsz * static_cast<int>(sizeof(T))>(vf, vb);
    }
  }
  // orders every later use of the tile's registers after the preceding wait
  template <bool E> __device__ void tie_all() {
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) tie<E>(kf[ks]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) tie<E>(vf[dt]);
  }
};

// Register-resident tile of 32 tokens of an FP8 cache: the same bytes per tile and the same
// load widths as a 16-token tile of 16-bit KV.  The QK product runs as two 16-row MFMA blocks;
// row r of block b is token 16b + r, so every key load reads whole 128-byte lines, and the two
// accumulators give lane (head, g) the scores of tokens 4g..4g+3 and 16+4g..16+4g+3.  Two row
// swaps move the probabilities to tokens 8g..8g+7 (compute32), the B operand of one 32-deep PV
// MFMA whose A operand is then 8 consecutive codes of one value dim (one 8-byte load).
//   kf[b][ks]: lane (row r16, g) holds 16-code key vector 4ks+g of token 16b + r16
//   vf[dt]:    lane (dim 16dt + r16, g) holds the codes of tokens 8g..8g+7
template <int D>
struct Tile32F8 {
  static constexpr int kTokens = 32;
  static constexpr int NK = D / 64;            // key vectors per lane and row block
  static constexpr int kLoads = 2 * NK + D / 16;
  u32x4 kf[2][NK];
  u32x2 vf[D / 16];

  template <int Bsz, bool E, bool NT, bool FLAT, bool MIX = false>
  __device__ void issue(const DecodeArgs& a, const int32_t* bt, int id_first, int ntok, const E4M3* kbase,
                        const E4M3* vbase, int t0, int64_t blk_stride, unsigned cached = 0) {
    constexpr int NB = 32 / Bsz;                 // blocks per tile: 4, 2 or 1
    constexpr int TPB = Bsz / 8;                 // 8-token groups per block
    const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
    const int first = t0 / Bsz;
    int id[NB];
    id[0] = FLAT ? id_first + first : (first == 0 ? id_first : ld_uniform(bt, first));
#pragma unroll
    for (int j = 1; j < NB; ++j) {
      id[j] = id[0];
      if (t0 + j * Bsz < ntok)   // later blocks of the tile, if any token is real
        id[j] = FLAT ? id_first + first + j : ld_uniform(bt, first + j);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) id[j] = min(max(id[j], 0), a.num_blocks - 1);
    // key rows: row r16 of block b is token 16b + r16.  Each load reads whole key lines (a block of
    // 16 rows holds 16 consecutive tokens of one 16-code vector), so it takes the stream's policy.
    // The previous row order (token 8(r/4) + 4b + r%4, which left the scores in the PV layout
    // directly) read every line in two 64-byte halves from two loads: 450 against 437 us on the
    // Llama-70B-class batch, where it had to keep key lines cacheable.
    const void* ka[2 * NK];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int tt = 16 * b + r16;
      const int jk = tt / Bsz;
      int bk = id[0];
#pragma unroll
      for (int j = 1; j < NB; ++j) bk = jk == j ? id[j] : bk;
      const E4M3* kb = kbase + static_cast<int64_t>(bk) * blk_stride + (g * Bsz + (tt & (Bsz - 1))) * 16;
      if constexpr (MIX && NK == 1) {
        ka[b] = kb;   // one load per row block: both row blocks in one group below
      } else if constexpr (MIX) {
        vload_group_strided<4 * Bsz * 16>(kf[b], kb, cached);
      } else {
        vload_strided<E, NT, 4 * Bsz * 16>(kf[b], kb);
      }
    }
    if constexpr (MIX && NK == 1) {
      u32x4(&kflat)[2 * NK] = *reinterpret_cast<u32x4(*)[2 * NK]>(&kf[0][0]);
      vload_group(kflat, ka, cached);
    }
    // value dims: tokens 8g..8g+7 lie in block g / TPB
    const int jv = g / TPB;
    int bv = id[0];
#pragma unroll
    for (int j = 1; j < NB; ++j) bv = jv == j ? id[j] : bv;
    const E4M3* vb = vbase + static_cast<int64_t>(bv) * blk_stride + r16 * Bsz + ((8 * g) & (Bsz - 1));
    if constexpr (MIX) {
      vload_group_strided<16 * Bsz>(vf, vb, cached);
    } else {
      vload_strided<E, NT, 16 * Bsz>(vf, vb);
    }
  }
  template <bool E> __device__ void tie_all() {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) tie<E>(kf[b][ks]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) tie<E>(vf[dt]);
  }
};

// q fragments of one query head hq of row s (q of type T, keys stored as KV): lane (r16, g)
// holds, in D / XQ / 4 16-byte vectors of XQ elements, the dims of the key vectors 4k+g its
// tile fragment holds (q vector j: the (j % R)-th XQ-element piece of key vector 4(j / R) + g,
// R = key elements per key vector / XQ, so 2 for 16-code FP8 key vectors and 16-bit q).
// kAsync: issued with vload (the caller waits explicitly); otherwise ordinary loads.
template <typename T, typename KV, int D, bool kAsync>
__device__ inline void load_q_head(const DecodeArgs& a, int s, int hq, u32x4* qr) {
  constexpr int XQ = 16 / sizeof(T);
  constexpr int R = Kv<KV>::X / XQ;
  const int g = threadIdx.x >> 4;
  const T* qrow = static_cast<const T*>(a.q) + (static_cast<int64_t>(s) * a.n_q_heads + hq) * D;
#pragma unroll
  for (int j = 0; j < D / XQ / 4; ++j) {
    const int dim0 = Kv<KV>::X * (4 * (j / R) + g) + XQ * (j % R);
    vload<kAsync, false>(qr[j], qrow + dim0);   // q rows are reread per partition
  }
}

// The LDS address (byte offset) of a __shared__ object.
template <typename P>
__device__ inline unsigned lds_offset(P* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) P*)p));
}

// 16 bytes per lane from g straight into LDS at lds_base + 16 * lane (a gfx950 global-to-LDS load):
// no register receives the data, and the load counts on vmcnt like any other, so a wait that retires
// a later load retires it too.  lds_base is wave-uniform.  M0, which holds the LDS address for the
// instruction, is saved and restored around it; the nop covers the M0 write before its use.
__device__ inline void lds_load16(const void* g, unsigned lds_base) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_base)
      : "memory");
}

// load_q_head into LDS: lane (r16, g)'s q vector j goes to dst[j][lane], as load_q_head puts it in
// qr[j] (the vectors of a head are NQ consecutive rows of 64 16-byte entries).
template <typename T, typename KV, int D>
__device__ inline void load_q_head_lds(const DecodeArgs& a, int s, int hq, u32x4 (*dst)[64]) {
  constexpr int XQ = 16 / sizeof(T);
  constexpr int R = Kv<KV>::X / XQ;
  const int g = threadIdx.x >> 4;
  const T* qrow = static_cast<const T*>(a.q) + (static_cast<int64_t>(s) * a.n_q_heads + hq) * D;
#pragma unroll
  for (int j = 0; j < D / XQ / 4; ++j) {
    const int dim0 = Kv<KV>::X * (4 * (j / R) + g) + XQ * (j % R);
    lds_load16(qrow + dim0, __builtin_amdgcn_readfirstlane(lds_offset(&dst[j][0])));
  }
}

// the X elements of a 16-byte vector as floats
template <typename T>
__device__ inline void unpack16(const u32x4& v, float* o) {
  if constexpr (sizeof(T) == 4) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y); o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  } else {
    T t[8];
    __builtin_memcpy(t, &v, 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = to_f32(t[e]);
  }
}
template <typename T, typename VV>
__device__ inline void unpack4(const VV& v, float* o) {
  T t[4];
  __builtin_memcpy(t, &v, 4 * sizeof(T));
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = to_f32(t[e]);
}

// ------------------------------------------------------------------------------ MFMA math
// PV on 16 tokens: O^T[16 dims][16 heads] += V^T[16 dims][16 tok] P^T[16 tok][16 heads]
__device__ inline f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c, __bf16) {
  s16x4 av, bv;
  __builtin_memcpy(&av, &a, 8);
  __builtin_memcpy(&bv, &b, 8);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, c, 0, 0, 0);
}
__device__ inline f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c, _Float16) {
  f16x4 av, bv;
  __builtin_memcpy(&av, &a, 8);
  __builtin_memcpy(&bv, &b, 8);
  return __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, c, 0, 0, 0);
}

// 4 E4M3 codes (a little-endian word) as 4 elements of T, exactly: every E4M3 value is
// representable in bf16 and in f16.  The packed gfx950 conversion with unit scale.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ inline u32x2 widen4(unsigned w, __bf16) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);   // codes 0, 1
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);    // codes 2, 3
  unsigned l, h;
  __builtin_memcpy(&l, &lo, 4);
  __builtin_memcpy(&h, &hi, 4);
  return u32x2{l, h};
}
__device__ inline u32x2 widen4(unsigned w, _Float16) {
  const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  unsigned l, h;
  __builtin_memcpy(&l, &lo, 4);
  __builtin_memcpy(&h, &hi, 4);
  return u32x2{l, h};
}
// 8 codes (two words) as the 8-element MFMA operand of type T
template <typename T>
__device__ inline typename Vec8<T>::type widen8(unsigned w0, unsigned w1) {
  const u32x2 a = widen4(w0, T{}), b = widen4(w1, T{});
  const u32x4 v = {a[0], a[1], b[0], b[1]};
  typename Vec8<T>::type r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// G <= 16 query heads of one KV head on 16-bit KV: S^T = K q^T (16 tokens x 16 heads, G of
// them real) and O^T += V^T P^T on MFMA.  The QK accumulator's lane layout (tokens 4g..4g+3
// for head lane%16) is the PV B operand, so the weights never leave their lanes; they are
// rounded to the KV type for the operand and the denominator sums the rounded values.
// KV = T: 16-bit keys and values; KV = E4M3: codes widened to T in registers, the key scale
// folded into scale_log2 by the caller and the value scale applied to the results.
template <typename T, int D, typename KV = T>
struct MfmaMath {
  static constexpr int QH = 1;            // q fragment sets parked per unit
  static constexpr bool kGroup = false;   // takes G from the kernel arguments
  static constexpr int NQ = D / 32;       // q vectors per lane: one per 32-wide MFMA k-step
  static constexpr bool kPrefetchQ = true;
  static constexpr bool kQuant = !std::is_same<KV, T>::value;
  using Tile = typename std::conditional<kQuant, Tile32F8<D>, Tile16<KV, D>>::type;
  f32x4 acc[D / 16];
  float m_run, l_run;

  __device__ void reset() {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // lanes of padded heads (h >= G) read head 0 of the group: their columns are discarded
  template <bool kAsync>
  __device__ static void load_q(const DecodeArgs& a, const Unit<KV>& u, u32x4 (*qr)[NQ]) {
    const int r16 = threadIdx.x & 15;
    load_q_head<T, KV, D, kAsync>(a, u.s, u.kvh * a.group + (r16 < a.group ? r16 : 0), qr[0]);
  }
  // the same fragments straight into a unit's LDS slot
  __device__ static void load_q_lds(const DecodeArgs& a, const Unit<KV>& u, u32x4 (*slot)[NQ][64]) {
    const int r16 = threadIdx.x & 15;
    load_q_head_lds<T, KV, D>(a, u.s, u.kvh * a.group + (r16 < a.group ? r16 : 0), slot[0]);
  }
  // Rescales the accumulators by alpha = 2^(old max - new max) when some lane's running max rose.
  // Otherwise every lane's alpha is exactly 1 (v_exp_f32 of 0), so skipping the multiply changes no
  // bit; once a row's leading tiles have passed the max rarely rises, and the skip saves reading each
  // accumulator out of its matrix-core registers, multiplying and writing it back on most tiles.
  __device__ void rescale(float alpha) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) == 0) return;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] = acc[dt] * alpha;
  }
  __device__ void compute(const Tile& R, const u32x4 (*q_lds)[NQ][64], int t0, int ntok, float scale_log2) {
    if constexpr (kQuant) compute32(R, q_lds, t0, ntok, scale_log2);
    else compute16(R, q_lds, t0, ntok, scale_log2);
  }
  // 16 tokens of 16-bit KV: S^T with one 16x16x32 MFMA per 32 dims, O^T += V^T P^T with 16x16x16
  __device__ void compute16(const Tile& R, const u32x4 (*q_lds)[NQ][64], int t0, int ntok, float scale_log2) {
    using V8 = typename Vec8<T>::type;
    const int g = threadIdx.x >> 4;
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const u32x4 qb = q_lds[0][j][threadIdx.x];
      V8 qv, kv;
      __builtin_memcpy(&qv, &qb, 16);
      __builtin_memcpy(&kv, &R.kf[j], 16);
      sc = mfma_16x16x32(kv, qv, sc);
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = sc[i] * scale_log2;
    const bool partial = t0 + 16 > ntok;
    if (partial) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + 4 * g + i >= ntok) x[i] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = max_x32(max_x16(mt));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    T pt[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pt[i] = static_cast<T>(fast_exp2(x[i] - m_new));
      psum += to_f32(pt[i]);
    }
    l_run = l_run * alpha + psum;
    rescale(alpha);
    u32x2 pb;
    __builtin_memcpy(&pb, pt, 8);
    // (the partial-tile test is taken once per tile, outside the value loop, so a full tile's value
    // products issue back to back)
    if (partial) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        u32x2 va = R.vf[dt];
        T vt[4];
        __builtin_memcpy(vt, &va, 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 4 * g + i >= ntok) vt[i] = static_cast<T>(0.f);
        __builtin_memcpy(&va, vt, 8);
        acc[dt] = mfma_16x16x16(va, pb, acc[dt], T{});
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt] = mfma_16x16x16(R.vf[dt], pb, acc[dt], T{});
    }
  }
  // 32 tokens of FP8 codes widened to T: two 16-row QK blocks per 32 dims, then one 32-deep
  // PV MFMA per 16 dims.  Lane (head r16, g) ends the QK product with the scores of tokens
  // 4g..4g+3 (block 0) and 16+4g..16+4g+3 (block 1); the softmax works in that layout (its
  // maxima and sums run over all four rows g), and two row swaps then hand the PV product the
  // weights of tokens 8g..8g+7.
  __device__ void compute32(const Tile& R, const u32x4 (*q_lds)[NQ][64], int t0, int ntok, float scale_log2) {
    using V8 = typename Vec8<T>::type;
    const int g = threadIdx.x >> 4;
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {   // key vector j / 2 holds 16 codes: q vector j takes half j % 2
      const u32x4 qb = q_lds[0][j][threadIdx.x];
      V8 qv;
      __builtin_memcpy(&qv, &qb, 16);
      const u32x4 k0 = R.kf[0][j / 2], k1 = R.kf[1][j / 2];
      const V8 a0 = (j % 2) ? widen8<T>(k0[2], k0[3]) : widen8<T>(k0[0], k0[1]);
      const V8 a1 = (j % 2) ? widen8<T>(k1[2], k1[3]) : widen8<T>(k1[0], k1[1]);
      s0 = mfma_16x16x32(a0, qv, s0);
      s1 = mfma_16x16x32(a1, qv, s1);
    }
    float x[8];   // tokens 4g + i (i < 4) and 16 + 4g + i - 4
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = s0[i] * scale_log2;
      x[4 + i] = s1[i] * scale_log2;
    }
    const bool partial = t0 + 32 > ntok;
    if (partial) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (t0 + (i < 4 ? 4 * g + i : 12 + 4 * g + i) >= ntok) x[i] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mt = max_x32(max_x16(mt));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    T pt[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pt[i] = static_cast<T>(fast_exp2(x[i] - m_new));
      psum += to_f32(pt[i]);
    }
    l_run = l_run * alpha + psum;
    rescale(alpha);
    // From the QK layout (pw[0..1]: tokens 4g..4g+3, pw[2..3]: tokens 16+4g..16+4g+3) to the PV
    // layout (tokens 8g..8g+7): the half swap gives rows g < 2 the first words of row g+2 as their
    // second words and rows g >= 2 the second words of row g-2 as their first; the row swap then
    // exchanges the second words of even rows with the first words of odd rows.
    unsigned pw[4];
    __builtin_memcpy(pw, pt, 16);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto r = __builtin_amdgcn_permlane32_swap(pw[w], pw[2 + w], false, false);
      pw[w] = r[0];
      pw[2 + w] = r[1];
    }
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto r = __builtin_amdgcn_permlane16_swap(pw[w], pw[2 + w], false, false);
      pw[w] = r[0];
      pw[2 + w] = r[1];
    }
    V8 pb;
    __builtin_memcpy(&pb, pw, 16);
    if (partial) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        V8 va = widen8<T>(R.vf[dt][0], R.vf[dt][1]);
        T vt[8];
        __builtin_memcpy(vt, &va, 16);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (t0 + 8 * g + i >= ntok) vt[i] = static_cast<T>(0.f);
        __builtin_memcpy(&va, vt, 16);
        acc[dt] = mfma_16x16x32(va, pb, acc[dt]);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt] = mfma_16x16x32(widen8<T>(R.vf[dt][0], R.vf[dt][1]), pb, acc[dt]);
    }
  }
  // A finished unit's results parked in LDS until the wave has no more units: the normalised
  // output of a one-partition row (part < 0), else the partition's (max, sum, accumulator).  For
  // groups of at most 8 heads: lane 16k + r holds head r, so lane r + 8g of an entry's 32 is
  // written by lane 16g + r.
  static constexpr bool kPark = true;
  struct Parked {
    f32x4 acc[D / 16][32];
    float m[8], l[8];
    int row0, part;
  };
  // the same values finish() stores, into LDS
  __device__ void park(const DecodeArgs& a, const Unit<KV>& u, Parked& p) {
    const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
    const float l_tot = sum_x32(sum_x16(l_run));
    if (threadIdx.x == 0) {
      p.row0 = u.s * a.n_q_heads + u.kvh * a.group;
      p.part = u.nparts == 1 ? -1 : u.part;
    }
    if (r16 >= 8) return;
    const float sc = u.nparts == 1 ? (kQuant ? a.v_scale / l_tot : 1.f / l_tot) : (kQuant ? a.v_scale : 1.f);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) p.acc[dt][8 * g + r16] = acc[dt] * sc;
    if (g == 0) {
      p.m[r16] = m_run;
      p.l[r16] = l_tot;
    }
  }
  // writes a parked unit's results where finish() would have
  __device__ static void unpark(const DecodeArgs& a, const Parked& p) {
    const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
    const int row0 = __builtin_amdgcn_readfirstlane(p.row0);
    const int part = __builtin_amdgcn_readfirstlane(p.part);
    if (r16 >= a.group) return;
    const int64_t row = row0 + r16;
    if (part < 0) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) store4<T>(a.out, row * D + 16 * dt + 4 * g, p.acc[dt][8 * g + r16], a.out_f32);
    } else {
      const int64_t pidx = row * a.max_parts + part;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) st_wt(a.part_acc + pidx * D + 16 * dt + 4 * g, p.acc[dt][8 * g + r16]);
      if (g == 0) {
        st_wt(a.part_m + pidx, p.m[r16]);
        st_wt(a.part_l + pidx, p.l[r16]);
      }
    }
  }
  // the normalised output when the row has one partition, else (max, sum, accumulator); with
  // quantised values the accumulator is scaled by the value scale
  __device__ void finish(const DecodeArgs& a, const Unit<KV>& u) {
    const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
    const float l_tot = sum_x32(sum_x16(l_run));
    if (r16 >= a.group) return;
    const int64_t row = static_cast<int64_t>(u.s) * a.n_q_heads + u.kvh * a.group + r16;
    if (u.nparts == 1) {
      const float inv = kQuant ? a.v_scale / l_tot : 1.f / l_tot;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) store4<T>(a.out, row * D + 16 * dt + 4 * g, acc[dt] * inv, a.out_f32);
    } else {
      const int64_t pidx = row * a.max_parts + u.part;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        st_wt(a.part_acc + pidx * D + 16 * dt + 4 * g, kQuant ? acc[dt] * a.v_scale : acc[dt]);
      if (g == 0) {
        st_wt(a.part_m + pidx, m_run);
        st_wt(a.part_l + pidx, l_tot);
      }
    }
  }
};

// ------------------------------------------------------------------------------ vector math
// G <= 4 query heads on fp32 KV (GM >= G): fp32 dot products per token (a lane's
// 4ks+g vectors, then a 4-lane cross-group reduction), softmax over the tile's 16 tokens with
// in-row reductions, fp32 weights, and FMA accumulation of the value columns (lane: dim
// 16dt + lane%16 over tokens 4g..4g+3, summed over the 4 groups when the unit ends).
template <typename T, int D, int GM>
struct VecMath {
  static constexpr bool kPark = false;   // results are stored as each unit ends
  struct Parked {};
  static constexpr int QH = GM;
  static constexpr bool kPrefetchQ = GM == 1;   // more heads: q is loaded at the unit switch
  static constexpr bool kGroup = true;
  using Tile = Tile16<T, D>;
  static constexpr int NQ = Tile::NK;
  static constexpr int X = Kv<T>::X;
  float acc[GM][D / 16];
  float m_run[GM], l_run[GM];
  int group;

  __device__ void reset() {
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      m_run[gi] = -INFINITY;
      l_run[gi] = 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[gi][dt] = 0.f;
    }
  }
  template <bool kAsync>
  __device__ static void load_q(const DecodeArgs& a, const Unit<T>& u, u32x4 (*qr)[NQ]) {
#pragma unroll
    for (int gi = 0; gi < GM; ++gi)
      load_q_head<T, T, D, kAsync>(a, u.s, u.kvh * a.group + (gi < a.group ? gi : 0), qr[gi]);
  }
  __device__ static void load_q_lds(const DecodeArgs& a, const Unit<T>& u, u32x4 (*slot)[NQ][64]) {
#pragma unroll
    for (int gi = 0; gi < GM; ++gi)
      load_q_head_lds<T, T, D>(a, u.s, u.kvh * a.group + (gi < a.group ? gi : 0), slot[gi]);
  }
  __device__ void compute(const Tile& R, const u32x4 (*q_lds)[NQ][64], int t0, int ntok, float scale_log2) {
    if constexpr (sizeof(T) == 4) compute_f32(R, q_lds, t0, ntok, scale_log2);
    else compute_16(R, q_lds, t0, ntok, scale_log2);
  }
  // fp32 KV: the tile's keys and values are read once as floats for all heads
  __device__ void compute_f32(const Tile& R, const u32x4 (*q_lds)[NQ][64], int t0, int ntok, float scale_log2) {
    const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
    const bool partial = t0 + 16 > ntok;
    float kv[Tile::NK][X];
#pragma unroll
    for (int ks = 0; ks < Tile::NK; ++ks) unpack16<T>(R.kf[ks], kv[ks]);
    float vv[D / 16][4];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      unpack4<T>(R.vf[dt], vv[dt]);
      if (partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 4 * g + i >= ntok) vv[dt][i] = 0.f;
      }
    }
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      if (gi >= group) break;
      float dot = 0.f;
#pragma unroll
      for (int ks = 0; ks < Tile::NK; ++ks) {
        float qv[X];
        unpack16<T>(q_lds[gi][ks][threadIdx.x], qv);
#pragma unroll
        for (int e = 0; e < X; ++e) dot = fmaf(qv[e], kv[ks][e], dot);
      }
      head_update(gi, dot, partial, r16, g, t0, ntok, scale_log2, [&](int dt, float* v4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = vv[dt][i];
      });
    }
  }
  // 16-bit KV (one head): each stored vector is widened to fp32 where it is used, so that no more than
  // one vector's floats are live at a time (widening the whole tile at once kept 64 more registers
  // live, which 16-bit tiles cannot afford next to the tile buffers)
  __device__ void compute_16(const Tile& R, const u32x4 (*q_lds)[NQ][64], int t0, int ntok, float scale_log2) {
    static_assert(GM == 1, "the 16-bit vector path takes one head per KV head");
    const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
    const bool partial = t0 + 16 > ntok;
    float dot = 0.f;
#pragma unroll
    for (int ks = 0; ks < Tile::NK; ++ks) {
      float kv[X], qv[X];
      unpack16<T>(R.kf[ks], kv);
      unpack16<T>(q_lds[0][ks][threadIdx.x], qv);
#pragma unroll
      for (int e = 0; e < X; ++e) dot = fmaf(qv[e], kv[e], dot);
    }
    head_update(0, dot, partial, r16, g, t0, ntok, scale_log2, [&](int dt, float* v4) {
      unpack4<T>(R.vf[dt], v4);
      if (partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 4 * g + i >= ntok) v4[i] = 0.f;
      }
    });
  }
  // head gi's share of a tile from the lane's partial dot product: the 4-lane reduction, the online
  // softmax over the tile's 16 tokens and the value accumulation (values_of(dt, v4): the lane's 4
  // tokens of value dim 16 dt + lane % 16, masked)
  template <class Values>
  __device__ void head_update(int gi, float dot, bool partial, int r16, int g, int t0, int ntok, float scale_log2,
                              Values values_of) {
    dot = sum_x32(sum_x16(dot));
    float xs = dot * scale_log2;
    if (partial && t0 + r16 >= ntok) xs = -INFINITY;
    float mt = fmaxf(xs, xor_f(xs, 1));
    mt = fmaxf(mt, xor_f(mt, 2));
    mt = fmaxf(mt, xor_f(mt, 4));
    mt = fmaxf(mt, xor_f(mt, 8));
    const float m_new = fmaxf(m_run[gi], mt);
    const float alpha = fast_exp2(m_run[gi] - m_new);
    m_run[gi] = m_new;
    const float p = fast_exp2(xs - m_new);    // weight of token t0 + r16
    l_run[gi] = l_run[gi] * alpha + (g == 0 ? p : 0.f);
    float pe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pe[i] = lane_fetch(p, 4 * g + i);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      float vv[4];
      values_of(dt, vv);
      float s4 = acc[gi][dt] * alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) s4 = fmaf(pe[i], vv[i], s4);
      acc[gi][dt] = s4;
    }
  }
  __device__ void finish(const DecodeArgs& a, const Unit<T>& u) {
    const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      if (gi >= group) break;
      float lt = l_run[gi];
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) lt += xor_f(lt, m);
      float o[D / 16];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        o[dt] = sum_x32(sum_x16(acc[gi][dt]));
      }
      if (g != 0) continue;
      const int64_t row = static_cast<int64_t>(u.s) * a.n_q_heads + u.kvh * a.group + gi;
      if (u.nparts == 1) {
        const float inv = 1.f / lt;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) store1<T>(a.out, row * D + 16 * dt + r16, o[dt] * inv, a.out_f32);
      } else {
        const int64_t pidx = row * a.max_parts + u.part;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) st_wt(a.part_acc + pidx * D + 16 * dt + r16, o[dt]);
        if (r16 == 0) {
          st_wt(a.part_m + pidx, m_run[gi]);
          st_wt(a.part_l + pidx, lt);
        }
      }
    }
  }
};

// ------------------------------------------------------------------------------ persistent kernel
// A wave claims its next unit with one atomic on the work counter; units are handed out in
// plan order, largest first.  Lane 0 alone executes the atomic: exec is narrowed inside the
// asm, so the result never passes through a divergent-branch merge that the compiler could
// copy before the value arrives.  The previous index in `slot` (lane 0) is valid once a wait
// covers the atomic; read it with readfirstlane.  Called with all lanes active (uniform
// control flow).
template <bool E>
__device__ inline void claim_unit(const DecodeArgs& a, int& slot) {
  if constexpr (!E) {
    int u = 0;
    if (threadIdx.x == 0) u = atomicAdd(&a.counters[1], 1);
    slot = u;
    return;
  }
  unsigned long long saved;
  asm volatile(
      "s_mov_b64 %1, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "global_atomic_add %0, %2, %3, off sc0\n\t"
      "s_mov_b64 exec, %1"
      : "=&v"(slot), "=&s"(saved)
      : "v"(a.counters + 1), "v"(1));
}

// Persistent wave over a stream of tiles of the units it claims, with NB tile buffers in rotation:
// while one tile is computed, the loads of the next NB - 1 are in flight.  The issue side runs up
// to one unit ahead of the compute side.  When it enters a unit it loads that unit's q straight
// into the unit's LDS slot (with kPrefetchQ; otherwise q is loaded when the compute side reaches
// the unit), before the unit's first tile loads, so the wait that retires that tile retires q too.
// When there is nothing left to issue it re-issues the current tile's loads (a filler the compute
// side skips), so each step issues the same loads on every path.
// The next unit is opened a few tiles before it is needed.  In the fixed rounds its index is known
// and nothing waits; after them the wave claims it from the counter and reads the claim after
// draining its loads, so the claim's result register never carries an in-flight value past that
// block (a claim read some steps later has its register moved by the register allocator under the
// pressure of five tile buffers, which the wait check reports).
// KV: the storage type of the pools (the tile's element); Math carries the compute type; NB: tile
// buffers; WPE: waves per SIMD the register budget is set for.
template <typename KV, int D, int Bsz, class Math, bool NT, bool FLAT, int NB, int WPE, bool MIX>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(WPE)))
void decode_kernel(DecodeArgs a) {
  using Tile = typename Math::Tile;
  constexpr int TT = Tile::kTokens;   // tokens per tile
  constexpr int NQ = Math::NQ;
  static_assert(NB >= 3 && NB <= 6, "tile buffers");
  // explicitly waited loads while the tile buffers fit in registers (32 per tile)
  constexpr bool E = sizeof(Tile) <= 32 * 4;
  static_assert(!MIX || (E && !NT), "a per-tile load policy needs the explicit waits");
  constexpr int LT = Tile::kLoads;   // every step issues exactly this many tile loads
  static_assert(!E || (NB - 1) * LT < 64, "vmcnt holds 6 bits");
  // q straight into LDS needs the explicit waits: the compiler's own waits do not know of such a load
  constexpr bool kQDma = Math::kPrefetchQ && E;
  constexpr int kClaimAhead = 4;   // take the next unit this many tiles before it is needed
  const int64_t chunk = static_cast<int64_t>(D) * Bsz;
  const int64_t blk_stride = chunk * a.n_kv_heads;
  const int total = ld_uniform(a.counters, 0) * a.n_kv_heads;
  __shared__ u32x4 q_lds[2][Math::QH][NQ][64];   // q fragments: compute unit's and issue unit's
  // Finished units' results wait in LDS while the wave reads on, and are written out when it has no
  // more units: result stores in the middle of the read stream slowed every wave (on the
  // Llama-70B-class batch the mean wave end fell 730 -> 717 us at P 3072 and 756 -> 722 us at
  // P 1536 once they moved to the end).  As many entries as fit beside q in this wave's share of
  // the CU's 160 KB; a unit that finds them full stores its results at once.  (FP8 pools in 8-token
  // blocks store at once: with parking, that kernel's register allocation failed the wait check.)
  using Parked = typename Math::Parked;
  constexpr int kLdsShare = 160 * 1024 / (4 * WPE);
  constexpr bool kParkHere = Math::kPark && !(sizeof(KV) == 1 && Bsz == 8);
  constexpr int NPARK = kParkHere ? static_cast<int>((kLdsShare - static_cast<int>(sizeof(q_lds)) - 512) /
                                                       static_cast<int>(sizeof(Parked)))
                                    : 0;
  __shared__ Parked parked[NPARK > 0 ? NPARK : 1];
  int n_parked = 0;

  // Each wave starts on one of the grid's first units, and the counter hands out the units after
  // them: every wave claiming its first unit from the one counter at once serialised 2048 atomics
  // and delayed the last waves' start (Llama-70B-class batch 789 -> 769 us, opt13b-class 146 ->
  // 126 us, swarm 118 -> 88 us once the first claims went).  Units are ordered longest first, so
  // the grid's first units are the ones the counter would have handed out first anyway.
  // Which first unit: workgroups are dispatched to the 8 XCDs in turn, so wave w runs on XCD w % 8.
  // Streamed (each block read by one row): XCD x starts on the x-th eighth of the units, every KV
  // head of consecutive (row, partition) pairs, so a row's table lines and blocks stay with one XCD
  // (1 % faster on the Llama-70B-class and opt13b-class batches).  Cacheable (blocks shared between
  // rows): wave w starts on unit w, KV head w % 8, so XCD x reads head x of every row and keeps the
  // shared blocks' lines of that head in its L2 (the other order made the swarm 14 % slower).
  const int grid = static_cast<int>(gridDim.x);
  const int first = (NT && !(grid & 7)) ? static_cast<int>((blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3))
                                        : static_cast<int>(blockIdx.x);
  // The first `rounds` units of every wave are fixed: round r gives wave w the unit at r * grid + first,
  // so a wave opens them with no claim.  Fixed rounds cover only full partitions (units of one size)
  // and at most three quarters of the units; the rest are handed out by the counter, which evens out
  // waves that ran slower.
  const int full_units = ld_uniform(a.counters, 17) * a.n_kv_heads;
  const int rounds = max(1, min(full_units / grid, (3 * total) / (4 * grid)));
  int round_i = 0;   // the fixed round of the issue cursor's unit
  if (first >= total) return;
  Unit<KV> uc = open_unit<KV, FLAT>(a, first, chunk);   // compute cursor
  Unit<KV> ui = uc;                              // issue cursor
  Unit<KV> un_next = uc;                         // the claimed unit after the issue cursor's
  u32x4 qr[Math::QH][NQ];
  auto park_q = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < Math::QH; ++h)
#pragma unroll
      for (int j = 0; j < NQ; ++j) q_lds[slot][h][j][threadIdx.x] = qr[h][j];
  };
  Math::template load_q<false>(a, uc, qr);   // the first unit's q: ordinary loads
  park_q(0);
  int slot_c = 0, slot_i = 0;
  // Wave-uniform state bits, packed in one word: separate flags captured by the lambdas below
  // get their stores merged through a pointer select, which puts them in scratch.
  constexpr unsigned kAhead = 1;    // the issue cursor is in the unit after the compute cursor's
  constexpr unsigned kEnded = 2;    // no more units to claim
  constexpr unsigned kNext = 16;    // un_next holds an opened unit the issue side has not reached
  unsigned fl = 0;
  int ti = 0, tc = 0;

  // Opens a claimed unit into un_next (its descriptor and first block id are dependent scalar reads,
  // done a few tiles before the switch instead of on its path); got: the counter value the claim
  // returned, read after a wait that retired it.
  auto open_index = [&](int un) __attribute__((always_inline)) {
    if (un >= 0 && un < total) {   // (a negative index can only be garbage: stop rather than fault)
      un_next = open_unit<KV, FLAT>(a, un, chunk);
      fl |= kNext;
    } else {
      fl |= kEnded;
    }
  };


  // Fills Y with the next tile of the issue stream; returns false when Y only holds filler
  // loads (nothing real left to issue right now) that the compute side must skip.
  // tc_now: the compute cursor's tile offset, passed by value (a reference capture keeps tc in memory).
  // Takes the wave's next unit into un_next: the next fixed round's unit, or after the fixed rounds one
  // from the counter.  A claim is read at once, after draining the wave's loads: the claim result's
  // register then holds an in-flight value only inside this block.
  auto take_next = [&]() __attribute__((always_inline)) {
    if (round_i + 1 < rounds) {
      ++round_i;
      open_index(round_i * grid + first);
    } else {
      int got = 0;
      claim_unit<E>(a, got);
      vm_wait<E, 0>();
      tie<E>(got);
      open_index(__builtin_amdgcn_readfirstlane(got) + rounds * grid);
    }
  };
  auto issue_next = [&](Tile& Y, int tc_now) __attribute__((always_inline)) -> bool {
    if (ti >= ui.ntok && !(fl & (kAhead | kEnded))) {
      if (!(fl & kNext)) take_next();   // a unit shorter than the look-ahead
      if (fl & kNext) {
        ui = un_next;
        ti = 0;
        fl = (fl | kAhead) & ~kNext;
        slot_i = slot_c ^ 1;
        // the unit's q goes straight into its LDS slot, ahead of the unit's first tile loads: the
        // compute side reads the slot only after the wait that retires that tile (slot_i belongs to
        // a unit the compute side has finished)
        if constexpr (kQDma) Math::load_q_lds(a, ui, q_lds[slot_i]);
      }
    }
    const bool is_real = ti < ui.ntok;
    // open the next unit a few tiles before it is needed (its descriptor is a dependent scalar load)
    if (is_real && !(fl & (kNext | kEnded)) && ui.ntok - (ti + TT) <= kClaimAhead * TT) take_next();
    // One load sequence on every path (a filler re-reads the compute cursor's tile, which keeps
    // the per-step loads uniform): separate sequences would meet in a merge that the compiler
    // may resolve by copying the loaded registers before the data arrives.
    // (unary + makes each operand a value: a select of lvalues selects their addresses, which
    // keeps the variables out of registers)
    // MIX: tiles that start in the rows' shared prefix are read cacheable, the others streamed
    unsigned cached = 0;
    if constexpr (MIX) {
      // (a filler's policy does not matter: the issue cursor's position decides it too)
      cached = __builtin_amdgcn_readfirstlane(ui.part * a.part_tokens + ti < a.cache_tokens ? 1 : 0);
    }
    Y.template issue<Bsz, E, NT, FLAT, MIX>(a, is_real ? +ui.bt : +uc.bt, is_real ? +ui.id_first : +uc.id_first,
                                      is_real ? +ui.ntok : +uc.ntok,
                                      static_cast<const KV*>(a.k_pool) + static_cast<int64_t>(is_real ? +ui.kvh : +uc.kvh) * chunk,
                                      static_cast<const KV*>(a.v_pool) + static_cast<int64_t>(is_real ? +ui.kvh : +uc.kvh) * chunk,
                                      is_real ? +ti : tc_now, blk_stride, cached);
    ti += is_real ? TT : 0;   // a select: a conditional update would put ti in memory
    return is_real;
  };

  Tile buf[NB] = {};   // defined before their first load, which names them as in/out operands
  // bit i set: buffer i holds a real tile of the compute unit, clear: a filler
  unsigned real = 0;
#pragma unroll
  for (int i = 0; i < NB - 1; ++i) real |= issue_next(buf[i], 0) ? (1u << i) : 0u;

  Math mt;
  mt.reset();
  if constexpr (Math::kGroup) mt.group = a.group;
  const float scale_log2 = a.scale_log2;

  // Step `xi` of the unrolled loop: computes buffer xi (issued NB - 1 steps ago) and issues the next
  // tile into buffer yi (computed one step ago).
  auto step = [&](auto xi, auto yi) __attribute__((always_inline)) -> bool {
    constexpr int XI = decltype(xi)::value, YI = decltype(yi)::value;
    constexpr unsigned XB = 1u << XI, YB = 1u << YI;
    Tile& X = buf[XI];
    const bool x_real = (real & XB) != 0;
    real = issue_next(buf[YI], tc) ? (real | YB) : (real & ~YB);
    // X was issued NB - 1 steps ago; each of the steps since issued LT tile loads
    vm_wait<E, (NB - 1) * LT>();
    X.template tie_all<E>();
    if (!x_real) return true;   // a filler: nothing to compute this step
    mt.compute(X, q_lds[slot_c], tc, uc.ntok, scale_log2);
    tc += TT;
    if (tc < uc.ntok) return true;
    if constexpr (NPARK > 0) {
      if (a.group <= 8 && n_parked < NPARK) {
        mt.park(a, uc, parked[n_parked]);
        ++n_parked;
      } else {
        mt.finish(a, uc);
      }
    } else {
      mt.finish(a, uc);
    }
    if (!(fl & kAhead)) return false;   // the issue side found no further unit: every issued tile is filler
    uc = ui;
    slot_c = slot_i;
    fl &= ~kAhead;
    tc = 0;
    mt.reset();
    if constexpr (!kQDma) {
      Math::template load_q<false>(a, uc, qr);   // the compiler waits for these itself
      park_q(slot_c);
    }
    return true;
  };
  // step i computes buffer i and issues into buffer i - 1 (mod NB)
  auto steps = [&](auto... is) __attribute__((always_inline)) {
    for (;;) {
      if (!(step(is, std::integral_constant<int, (decltype(is)::value + NB - 1) % NB>{}) && ...)) break;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  if constexpr (NB == 3) steps(I0{}, I1{}, I2{});
  else if constexpr (NB == 4) steps(I0{}, I1{}, I2{}, I3{});
  else if constexpr (NB == 5) steps(I0{}, I1{}, I2{}, I3{}, I4{});
  else steps(I0{}, I1{}, I2{}, I3{}, I4{}, I5{});
  vm_wait<E, 0>();   // filler loads still in flight land before the wave ends
  if constexpr (NPARK > 0) {
    for (int k = 0; k < n_parked; ++k) Math::unpark(a, parked[k]);
  }
}

// ------------------------------------------------------------------------------ merge
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p with M = max_p m_p, for rows with more
// than one partition.  One wave per (row, query head), four heads per workgroup.  M comes first
// (one load of the partitions' maxima across the lanes, then a wave maximum); then every
// partition's weight is known and the accumulator loads (D/64 consecutive floats per lane) are
// independent of each other, eight in flight at once.  Measured against four waves per head
// (every 4th partition each, combined in LDS): 12.3 against 20.3 us on the Llama-70B-class batch
// (2-3 partitions a row), 7.0 against 6.3 us on 64 k-token rows (32 partitions).
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;  // output elements per lane
  const int s = blockIdx.x;
  const int head = blockIdx.y * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int L = row_len(a, s);
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1 || head >= a.n_q_heads) return;
  const int64_t pbase = (static_cast<int64_t>(s) * a.n_q_heads + head) * a.max_parts;
  const float* pm = a.part_m + pbase;
  const float* pl = a.part_l + pbase;
  float M = -INFINITY;   // lane p holds partitions p, p + 64, ...; then a wave maximum
  for (int p = lane; p < np; p += 64) M = fmaxf(M, pm[p]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, xor_f(M, d));
  float den = 0.f, num[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) num[i] = 0.f;
#pragma unroll 8
  for (int p = 0; p < np; ++p) {
    const float w = fast_exp2(pm[p] - M);
    float v[PER];
    if constexpr (PER == 2) {
      const float2 t = *reinterpret_cast<const float2*>(a.part_acc + (pbase + p) * D + 2 * lane);
      v[0] = t.x;
      v[1] = t.y;
    } else {
      v[0] = a.part_acc[(pbase + p) * D + lane];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) num[i] = fmaf(w, v[i], num[i]);
    den = fmaf(w, pl[p], den);
  }
  const float inv = 1.f / den;
  const int64_t row = static_cast<int64_t>(s) * a.n_q_heads + head;
#pragma unroll
  for (int i = 0; i < PER; ++i) store1<T>(a.out, row * D + PER * lane + i, num[i] * inv, a.out_f32);
}

// ------------------------------------------------------------------------------ dispatch
// Tile buffers and waves per SIMD of each kernel variant.  Streamed 16-bit pools: five buffers, one
// wave per SIMD (measured on the Llama-70B-class batch: 753-756 us per decode call against 761-766 us
// with three buffers and two waves per SIMD; the MHA batch 123 against 127 us).  Streamed FP8 pools:
// four (five do not fit beside the widening registers).  Cacheable and per-tile-policy loads (batches
// whose rows share blocks), and fp32 pools: three buffers, two waves per SIMD, for the wider grid that
// a batch of few long rows needs (the 20-row shared-prompt batch, every tile streamed: 92 us with three
// buffers and two waves per SIMD against 116 us with five and one).  The defaults may be overridden at
// compile time to measure other depths.
#ifndef PKV_NB16
#define PKV_NB16 5
#endif
#ifndef PKV_WPE16
#define PKV_WPE16 1
#endif
#ifndef PKV_NB8
#define PKV_NB8 4
#endif
#ifndef PKV_WPE8
#define PKV_WPE8 1
#endif
template <typename KV, class Math, bool NT> struct Pipeline {
  static constexpr bool k16 = sizeof(KV) == 2 && NT;   // streamed 16-bit pools on MFMA
  static constexpr bool k8 = std::is_same<KV, E4M3>::value && NT;
  static constexpr int NB = k16 ? PKV_NB16 : k8 ? PKV_NB8 : 3;
  static constexpr int WPE = k16 ? PKV_WPE16 : k8 ? PKV_WPE8 : 2;
};

template <typename KV, int D, class Math, bool NT, bool FLAT = false, bool MIX = false>
const void* kernel_ptr_b(int block_size) {
  constexpr int NB = Pipeline<KV, Math, NT>::NB, W = Pipeline<KV, Math, NT>::WPE;
  switch (block_size) {
    case 8: return reinterpret_cast<const void*>(&decode_kernel<KV, D, 8, Math, NT, FLAT, NB, W, MIX>);
    case 16: return reinterpret_cast<const void*>(&decode_kernel<KV, D, 16, Math, NT, FLAT, NB, W, MIX>);
    case 32: return reinterpret_cast<const void*>(&decode_kernel<KV, D, 32, Math, NT, FLAT, NB, W, MIX>);
    default: return nullptr;
  }
}

// T: the type of q and of the outputs; fp8: the pools hold E4M3 codes (MFMA path only); flat: rows
// read consecutive blocks of their span (16-bit KV on MFMA, streamed loads only)
template <typename T, int D>
const void* kernel_ptr_d(int path, int group, int block_size, int pol, bool fp8, bool flat) {
  const bool nt = pol == kLoadStreamed, mix = pol == kLoadMixed;
  if (flat) {
    if constexpr (sizeof(T) == 2)
      if (path == 1 && !fp8 && nt) return kernel_ptr_b<T, D, MfmaMath<T, D>, true, true>(block_size);
    return nullptr;
  }
  if (path == 1) {
    if constexpr (sizeof(T) == 2) {
      if (fp8)
        return nt ? kernel_ptr_b<E4M3, D, MfmaMath<T, D, E4M3>, true>(block_size)
               : mix ? kernel_ptr_b<E4M3, D, MfmaMath<T, D, E4M3>, false, false, true>(block_size)
                     : kernel_ptr_b<E4M3, D, MfmaMath<T, D, E4M3>, false>(block_size);
      return nt ? kernel_ptr_b<T, D, MfmaMath<T, D>, true>(block_size)
             : mix ? kernel_ptr_b<T, D, MfmaMath<T, D>, false, false, true>(block_size)
                   : kernel_ptr_b<T, D, MfmaMath<T, D>, false>(block_size);
    }
    return nullptr;
  }
  if (fp8 || mix) return nullptr;
  // the vector path: fp32 KV (always streamed), and 16-bit KV with G = 1 when the caller asks for it
  if constexpr (sizeof(T) == 4) {
    if (group == 1) return kernel_ptr_b<T, D, VecMath<T, D, 1>, true>(block_size);
    if (group == 2) return kernel_ptr_b<T, D, VecMath<T, D, 2>, true>(block_size);
    return kernel_ptr_b<T, D, VecMath<T, D, 4>, true>(block_size);
  } else {
    if (group == 1)
      return nt ? kernel_ptr_b<T, D, VecMath<T, D, 1>, true>(block_size)
                : kernel_ptr_b<T, D, VecMath<T, D, 1>, false>(block_size);
    return nullptr;
  }
}

template <typename T>
const void* main_kernel_ptr(int head_dim, int path, int group, int block_size, int pol, bool fp8, bool flat) {
  return head_dim == 128 ? kernel_ptr_d<T, 128>(path, group, block_size, pol, fp8, flat)
                         : kernel_ptr_d<T, 64>(path, group, block_size, pol, fp8, flat);
}

template <typename T, int D>
void reduce_launch(const DecodeArgs& a, hipStream_t st) {
  decode_reduce_kernel<T, D><<<dim3(a.num_seqs, (a.n_q_heads + 3) / 4), dim3(256), 0, st>>>(a);
}

}  // namespace

hipError_t launch_decode_plan(const DecodeArgs& a, int dtype, int head_dim, hipStream_t st) {
  if (dtype == PKV_F32) decode_plan_kernel<float><<<1, 1024, 0, st>>>(a, head_dim);
  else if (dtype == PKV_F16) decode_plan_kernel<_Float16><<<1, 1024, 0, st>>>(a, head_dim);
  else decode_plan_kernel<__bf16><<<1, 1024, 0, st>>>(a, head_dim);
  return hipGetLastError();
}

hipError_t launch_step_prologue(const DecodeArgs& a, const ScatterArgs& sc, const StepArgs& sa, int dtype,
                                bool kv_fp8, int head_dim, hipStream_t st) {
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;   // the LDS slot stage assumes it
  const int elem = kv_fp8 ? 16 : (dtype == PKV_F32 ? 4 : 8);             // elements per 16-byte key vector
  const int64_t vectors = static_cast<int64_t>(sc.num_tokens) * sc.n_kv_heads * (sc.head_dim / elem);
  const int64_t blocks = 1 + (vectors + 255) / 256;                     // 256 vectors per scatter workgroup
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grd(static_cast<unsigned>(blocks)), blk(1024);
  if (dtype == PKV_F32) {
    if (kv_fp8) return hipErrorInvalidValue;   // a quantised cache takes 16-bit rows and queries
    step_prologue_kernel<float, false><<<grd, blk, 0, st>>>(a, sc, sa, head_dim);
  } else if (dtype == PKV_F16) {
    if (kv_fp8) step_prologue_kernel<_Float16, true><<<grd, blk, 0, st>>>(a, sc, sa, head_dim);
    else step_prologue_kernel<_Float16, false><<<grd, blk, 0, st>>>(a, sc, sa, head_dim);
  } else {
    if (kv_fp8) step_prologue_kernel<__bf16, true><<<grd, blk, 0, st>>>(a, sc, sa, head_dim);
    else step_prologue_kernel<__bf16, false><<<grd, blk, 0, st>>>(a, sc, sa, head_dim);
  }
  return hipGetLastError();
}

hipError_t launch_decode_main(const DecodeArgs& a, int dtype, bool kv_fp8, int head_dim, int path, int pol,
                              int32_t grid, hipStream_t st) {
  const bool flat = a.flat_bps > 0;
  const void* fn =
      dtype == PKV_F32   ? main_kernel_ptr<float>(head_dim, path, a.group, a.block_size, pol, kv_fp8, flat)
      : dtype == PKV_F16 ? main_kernel_ptr<_Float16>(head_dim, path, a.group, a.block_size, pol, kv_fp8, flat)
                         : main_kernel_ptr<__bf16>(head_dim, path, a.group, a.block_size, pol, kv_fp8, flat);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(grid), dim3(64), args, 0, st);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim, hipStream_t st) {
  if (dtype == PKV_F32) {
    if (head_dim == 128) reduce_launch<float, 128>(a, st);
    else reduce_launch<float, 64>(a, st);
  } else if (dtype == PKV_F16) {
    if (head_dim == 128) reduce_launch<_Float16, 128>(a, st);
    else reduce_launch<_Float16, 64>(a, st);
  } else {
    if (head_dim == 128) reduce_launch<__bf16, 128>(a, st);
    else reduce_launch<__bf16, 64>(a, st);
  }
  return hipGetLastError();
}

hipError_t decode_main_grid_cap(int dtype, bool kv_fp8, bool flat, int head_dim, int path, int group,
                                int block_size, int pol, int32_t* cap) {
  // the load policies have their own pipeline shapes, so their own occupancy
  const void* fn =
      dtype == PKV_F32   ? main_kernel_ptr<float>(head_dim, path, group, block_size, pol, kv_fp8, flat)
      : dtype == PKV_F16 ? main_kernel_ptr<_Float16>(head_dim, path, group, block_size, pol, kv_fp8, flat)
                         : main_kernel_ptr<__bf16>(head_dim, path, group, block_size, pol, kv_fp8, flat);
  if (!fn) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  *cap = cus * per_cu;
  return hipSuccess;
}

}  // namespace pkv
