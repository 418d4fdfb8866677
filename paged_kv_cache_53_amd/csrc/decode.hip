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
//   plan kernel lists the (row, partition) pairs; a persistent grid of
//   single-wave workgroups takes units from an atomic counter, so no
//   workgroup is launched for a partition that does not exist and long and
//   short rows balance across the 256 CUs.
// * A wave walks its partition in tiles of 32 tokens (MFMA path) or 16 tokens
//   (vector path).  The partition's block ids are read once, one per lane,
//   and each lane picks the id of its token's block with ds_bpermute.
// * Key rows are stored as 16-byte vectors [c][token][X]: the 64 lanes of a
//   wave read 1 KiB contiguous per load (lane = token within 16, lane group =
//   vector column).  Values are stored [dim][token] so that a lane's 4 or 8
//   consecutive tokens of one dimension are one 8- or 16-byte load -- exactly
//   the operand the PV product contracts over.
// * MFMA path (16-bit KV, G >= 4): S^T = K q^T and O^T = V^T P^T with
//   v_mfma_f32_16x16x32_{bf16,f16}; the G query heads of a KV head are the
//   16-wide N dimension (zero-padded).  The QK accumulator layout (lane holds
//   tokens 4g..4g+3 of each 16-token half for head lane%16) is exactly the B
//   operand layout of the PV product, so weights never leave their lanes.
//   The weights are rounded to the KV type for the PV operand, and the
//   denominator sums the rounded values.
// * Vector path (fp32 KV, or G < 4): per-token dot products with a 4-lane
//   cross-group reduction, fp32 weights, FMA accumulation.
// * Online softmax in the base-2 domain (scores pre-multiplied by
//   scale*log2(e), v_exp_f32); masked tokens get -inf scores and zeroed value
//   elements (selected, never multiplied, so a NaN in an unused slot cannot
//   leak in).  Rows with one partition write the output directly; longer rows
//   write (max, sum, acc) partials that the reduce kernel merges.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
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

template <typename T> __device__ inline float to_f32(T x) { return static_cast<float>(x); }

// Stores 4 consecutive output elements.
template <typename T>
__device__ inline void store4(void* out, int64_t idx, f32x4 v, bool f32out) {
  if (f32out) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = v;
  } else {
    T t[4] = {static_cast<T>(v[0]), static_cast<T>(v[1]), static_cast<T>(v[2]), static_cast<T>(v[3])};
    uint2 bits;
    __builtin_memcpy(&bits, t, 8);
    *reinterpret_cast<uint2*>(static_cast<T*>(out) + idx) = bits;
  }
}
template <typename T>
__device__ inline void store1(void* out, int64_t idx, float v, bool f32out) {
  if (f32out) static_cast<float*>(out)[idx] = v;
  else static_cast<T*>(out)[idx] = static_cast<T>(v);
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

// Next unit for this wave, or -1 when the list is exhausted.
__device__ inline int next_unit(const DecodeArgs& a, int total) {
  int u = 0;
  if (threadIdx.x == 0) u = atomicAdd(&a.counters[1], 1);
  u = __builtin_amdgcn_readfirstlane(u);
  return u < total ? u : -1;
}

// ------------------------------------------------------------------------------ plan
// Lists the (row, partition) pairs, largest first: every full partition, then each row's
// shorter last partition in decreasing length (counting sort over 16-token buckets).  Waves
// claim units in this order, so the last units handed out are the shortest and the waves
// finish together.  The order decides only which wave computes a unit, never its result.
template <typename T>
__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a, int head_dim) {
  constexpr int NBUCKET = 1024;
  __shared__ int sums[1024];
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
    const int L = row_len(a, s);
    full_local += L / P;
    if (L % P) atomicAdd(&bucket_fill[((L % P) - 1) >> shift], 1);
  }
  sums[tid] = full_local;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? sums[tid - d] : 0;
    __syncthreads();
    sums[tid] += v;
    __syncthreads();
  }
  const int full_total = sums[1023];
  // bucket bases, longest bucket first, after all full partitions (one thread: <= 1024 adds)
  if (tid == 0) {
    int acc = full_total;
    for (int bk = NBUCKET - 1; bk >= 0; --bk) {
      bucket_base[bk] = acc;
      acc += bucket_fill[bk];
      bucket_fill[bk] = 0;
    }
    a.counters[0] = acc;
  }
  __syncthreads();
  int off = sums[tid] - full_local;
  const int64_t row_elems = static_cast<int64_t>(a.n_q_heads) * head_dim;
  for (int s = lo; s < hi; ++s) {
    const int L = row_len(a, s);
    const int nfull = L / P;
    for (int p = 0; p < nfull; ++p) a.units[off + p] = make_int2(s, p);
    off += nfull;
    if (L % P) {
      const int bk = ((L % P) - 1) >> shift;
      a.units[bucket_base[bk] + atomicAdd(&bucket_fill[bk], 1)] = make_int2(s, nfull);
    }
    if (L == 0) {  // empty row: zeros
      for (int64_t i = 0; i < row_elems; ++i) store1<T>(a.out, s * row_elems + i, 0.f, a.out_f32);
    }
  }
  if (tid >= 1 && tid <= 16) a.counters[tid] = 0;   // work-claim counters
}

// ------------------------------------------------------------------------------ MFMA path
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

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

// Register-resident tile of 16 tokens: the key rows in the A-operand layout of the QK
// product (lane: token lane%16, 16-byte vectors 4ks+lane/16), the value columns in the
// A-operand layout of the PV product (lane: dim 16dt+lane%16, tokens 4(lane/16)..+3).
template <int D>
struct Tile16 {
  u32x4 kf[D / 32];
  u32x2 vf[D / 16];
};

// One work unit (row s, KV head kvh, partition part); all fields are wave-uniform.
template <typename T>
struct Unit {
  int s, kvh, part, ntok, nparts;
  const int32_t* bt;  // block-table row at the partition's first block
  const T* kbase;     // k_pool + kvh * chunk
  const T* vbase;
};

template <typename T>
__device__ inline Unit<T> open_unit(const DecodeArgs& a, int id, int64_t chunk) {
  Unit<T> u;
  const int pair = id / a.n_kv_heads;
  u.kvh = id - pair * a.n_kv_heads;
  u.s = ld_uniform(reinterpret_cast<const int32_t*>(a.units), 2 * static_cast<int64_t>(pair));
  u.part = ld_uniform(reinterpret_cast<const int32_t*>(a.units), 2 * static_cast<int64_t>(pair) + 1);
  const int L = row_len(a, u.s);
  const int tok0 = u.part * a.part_tokens;
  u.ntok = min(a.part_tokens, L - tok0);
  u.nparts = (L + a.part_tokens - 1) / a.part_tokens;
  u.bt = a.block_tables + static_cast<int64_t>(u.s) * a.bt_stride + (tok0 >> a.log2_block);
  u.kbase = static_cast<const T*>(a.k_pool) + static_cast<int64_t>(u.kvh) * chunk;
  u.vbase = static_cast<const T*>(a.v_pool) + static_cast<int64_t>(u.kvh) * chunk;
  return u;
}

// q^T as the B operand of S^T = K q^T: lane (g, h) holds q[h][8*(4ks+g) .. +8].  Lanes of
// padded heads (h >= G) read head 0 of the group: their columns are computed and discarded.
template <typename T, int D>
__device__ inline void load_q(const DecodeArgs& a, const Unit<T>& u, u32x4 (&qr)[D / 32]) {
  const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int h = r16 < a.group ? r16 : 0;
  const T* qrow = static_cast<const T*>(a.q) + (static_cast<int64_t>(u.s) * a.n_q_heads + u.kvh * a.group + h) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qr[ks] = *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * ks + g));
}

// Issues the loads of the 16-token tile at partition offset t0 of unit u.  Block ids are
// wave-uniform scalar loads; table entries past the unit's last block are never read (those
// tokens reuse the first id and are masked in the compute).
template <typename T, int D, int Bsz>
__device__ inline void issue_tile(const DecodeArgs& a, const Unit<T>& u, int t0, int64_t blk_stride,
                                  Tile16<D>& R) {
  constexpr int X = 8;
  constexpr int NB = Bsz >= 16 ? 1 : 16 / Bsz;   // blocks per tile
  const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int first = t0 / Bsz;
  int id0 = ld_uniform(u.bt, first);
  id0 = min(max(id0, 0), a.num_blocks - 1);
  int id1 = id0;
  if constexpr (NB == 2) {
    if (t0 + 8 < u.ntok) {
      id1 = ld_uniform(u.bt, first + 1);
      id1 = min(max(id1, 0), a.num_blocks - 1);
    }
  }
  const int bk = (NB == 2 && r16 >= 8) ? id1 : id0;
  const T* kb = u.kbase + static_cast<int64_t>(bk) * blk_stride + (((t0 + r16) & (Bsz - 1)) + g * Bsz) * X;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    R.kf[ks] = *reinterpret_cast<const u32x4*>(kb + ks * 4 * Bsz * X);
  const int bv = (NB == 2 && g >= 2) ? id1 : id0;
  const T* vb = u.vbase + static_cast<int64_t>(bv) * blk_stride + r16 * Bsz + ((t0 + 4 * g) & (Bsz - 1));
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    R.vf[dt] = *reinterpret_cast<const u32x2*>(vb + dt * 16 * Bsz);
}

// QK^T, online softmax (base 2) and PV of one loaded 16-token tile.
template <typename T, int D>
__device__ inline void compute_tile(const Tile16<D>& R, const u32x4 (*q_lds)[64], int t0, int ntok,
                                    float scale_log2, float& m_run, float& l_run, f32x4 (&acc)[D / 16]) {
  using V8 = typename Vec8<T>::type;
  const int g = threadIdx.x >> 4;
  f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const u32x4 qb = q_lds[ks][threadIdx.x];
    V8 qv, kv;
    __builtin_memcpy(&qv, &qb, 16);
    __builtin_memcpy(&kv, &R.kf[ks], 16);
    sc = mfma_16x16x32(kv, qv, sc);
  }
  // lane (g, h) holds the scores of tokens t0 + 4g + i, i = 0..3, for head h
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
  mt = fmaxf(mt, xor_f(mt, 16));
  mt = fmaxf(mt, xor_f(mt, 32));
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
  u32x2 pb;
  __builtin_memcpy(&pb, pt, 8);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    u32x2 va = R.vf[dt];
    if (partial) {
      T vt[4];
      __builtin_memcpy(vt, &va, 8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + 4 * g + i >= ntok) vt[i] = static_cast<T>(0.f);
      __builtin_memcpy(&va, vt, 8);
    }
    acc[dt] = mfma_16x16x16(va, pb, acc[dt] * alpha, T{});
  }
}

// Writes a finished unit: the normalised output when the row has one partition, else the
// partition's (max, sum, unnormalised accumulator) for the merge kernel.
template <typename T, int D>
__device__ inline void finish_unit(const DecodeArgs& a, const Unit<T>& u, float m_run, float l_run,
                                   const f32x4 (&acc)[D / 16]) {
  const int r16 = threadIdx.x & 15, g = threadIdx.x >> 4;
  float l_tot = l_run + xor_f(l_run, 16);
  l_tot += xor_f(l_tot, 32);
  if (r16 >= a.group) return;
  const int64_t row = static_cast<int64_t>(u.s) * a.n_q_heads + u.kvh * a.group + r16;
  if (u.nparts == 1) {
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) store4<T>(a.out, row * D + 16 * dt + 4 * g, acc[dt] * inv, a.out_f32);
  } else {
    const int64_t pidx = row * a.max_parts + u.part;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<f32x4*>(a.part_acc + pidx * D + 16 * dt + 4 * g) = acc[dt];
    if (g == 0) {
      a.part_m[pidx] = m_run;
      a.part_l[pidx] = l_tot;
    }
  }
}

// A wave claims its next unit with one atomic on the work counter (lane 0); units are handed
// out in plan order, largest first.
__device__ inline int claim_unit(const DecodeArgs& a) {
  int u = 0;
  if (threadIdx.x == 0) u = atomicAdd(&a.counters[1], 1);
  return u;  // valid in lane 0 only; read with readfirstlane when needed
}

// Persistent wave over a stream of 16-token tiles of the units it claims, with the loads of
// the tile two steps ahead in flight while the current tile is computed (three tile buffers
// in rotation).  The issue side runs up to one unit ahead of the compute side; it loads that
// unit's q into registers before the unit's first tile loads and parks it in the unit's LDS
// slot one step later, after that step's tile loads are issued, so every wait in the steady
// state covers exactly the tile about to be used.  When there is nothing left to issue it
// re-issues the current tile's loads, so each step issues the same loads on every path.
template <typename T, int D, int Bsz>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_kernel(DecodeArgs a) {
  const int64_t chunk = static_cast<int64_t>(D) * Bsz;
  const int64_t blk_stride = chunk * a.n_kv_heads;
  const int total = ld_uniform(a.counters, 0) * a.n_kv_heads;
  __shared__ u32x4 q_lds[2][D / 32][64];   // q fragments of the compute unit and the issue unit

  const int first = __builtin_amdgcn_readfirstlane(claim_unit(a));
  if (first >= total) return;
  Unit<T> uc = open_unit<T>(a, first, chunk);   // compute cursor
  Unit<T> ui = uc;                              // issue cursor
  u32x4 qr[D / 32];
  load_q<T, D>(a, uc, qr);
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) q_lds[0][ks][threadIdx.x] = qr[ks];
  int slot_c = 0, slot_i = 0;
  bool ahead = false;        // the issue cursor is in the unit after the compute cursor's
  bool ended = false;        // no more units to claim
  bool q_pending = false;    // qr holds the issue unit's q, not yet parked
  int pending = 0;
  bool claimed = false;      // `pending` holds a claim whose result is not read yet
  int ti = 0, tc = 0;
  constexpr int kClaimAhead = 4;   // claim the next unit this many tiles before it is needed

  // Fills Y with the next tile of the issue stream; returns false when Y only holds filler
  // loads (nothing real left to issue right now) that the compute side must skip.
  auto issue_next = [&](Tile16<D>& Y) __attribute__((always_inline)) -> bool {
    if (ti >= ui.ntok && !ahead && !ended) {
      if (!claimed) pending = claim_unit(a);
      const int un = __builtin_amdgcn_readfirstlane(pending);
      claimed = false;
      if (un < total) {
        ui = open_unit<T>(a, un, chunk);
        ti = 0;
        ahead = true;
        slot_i = slot_c ^ 1;
        load_q<T, D>(a, ui, qr);
        q_pending = true;
      } else {
        ended = true;
      }
    }
    if (ti < ui.ntok) {
      issue_tile<T, D, Bsz>(a, ui, ti, blk_stride, Y);
      ti += 16;
      if (!claimed && !ended && ui.ntok - ti <= kClaimAhead * 16) {
        pending = claim_unit(a);
        claimed = true;
      }
      return true;
    }
    issue_tile<T, D, Bsz>(a, uc, tc, blk_stride, Y);   // filler: keeps the per-step loads uniform
    return false;
  };

  Tile16<D> A, B, C;
  bool rA = issue_next(A);
  bool rB = issue_next(B);
  bool rC = false;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // X: the buffer issued two steps ago (rX: it holds a real tile of uc); Y gets the next issue.
  auto step = [&](Tile16<D>& X, bool& rX, Tile16<D>& Y, bool& rY) __attribute__((always_inline)) -> bool {
    if (q_pending) {   // loaded a step ago, before that step's tile loads
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) q_lds[slot_i][ks][threadIdx.x] = qr[ks];
      q_pending = false;
    }
    rY = issue_next(Y);
    if (!rX) return true;   // a filler: nothing to compute this step
    compute_tile<T, D>(X, q_lds[slot_c], tc, uc.ntok, a.scale_log2, m_run, l_run, acc);
    tc += 16;
    if (tc < uc.ntok) return true;
    finish_unit<T, D>(a, uc, m_run, l_run, acc);
    if (!ahead) return false;   // the issue side found no further unit: every issued tile is filler
    uc = ui;
    slot_c = slot_i;
    ahead = false;
    tc = 0;
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    return true;
  };
  for (;;) {
    if (!step(A, rA, C, rC)) break;
    if (!step(B, rB, A, rA)) break;
    if (!step(C, rC, B, rB)) break;
  }
}

// ------------------------------------------------------------------------------ vector path
template <typename T, int D, int GM>
__global__ __launch_bounds__(64) void decode_vec_kernel(DecodeArgs a) {
  constexpr int X = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte vector
  constexpr int C = D / X;                              // vectors per key row
  constexpr int KC = C / 4;                             // vectors per lane per token
  constexpr int PPR = static_cast<int>(sizeof(T));      // 16-byte parts of a 16-token value row
  constexpr int RSTEP = 64 / PPR;                       // rows covered per load instruction
  constexpr int RPL = D / RSTEP;                        // value rows per lane
  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int vrow = lane / PPR;
  const int vpart = lane % PPR;
  const int Hk = a.n_kv_heads;
  const int G = a.group;
  const int Bsz = a.block_size;
  const int lb = a.log2_block;
  const int64_t chunk = static_cast<int64_t>(D) * Bsz;
  const int64_t blk_stride = chunk * Hk;
  const T* __restrict__ kpool = static_cast<const T*>(a.k_pool);
  const T* __restrict__ vpool = static_cast<const T*>(a.v_pool);
  const int total = a.counters[0] * Hk;

  for (int u = next_unit(a, total); u >= 0; u = next_unit(a, total)) {
    const int pair = u / Hk;
    const int kvh = u - pair * Hk;
    const int2 sp = a.units[pair];
    const int s = sp.x;
    const int part = sp.y;
    const int L = row_len(a, s);
    const int tok0 = part * a.part_tokens;
    const int ntok = min(a.part_tokens, L - tok0);
    const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
    const int32_t* bt = a.block_tables + static_cast<int64_t>(s) * a.bt_stride + (tok0 >> lb);
    const int nblk = (ntok + Bsz - 1) >> lb;
    const T* kbase = kpool + static_cast<int64_t>(kvh) * chunk;
    const T* vbase = vpool + static_cast<int64_t>(kvh) * chunk;

    // q slices matching this lane's key vectors c = 4*kc + g
    float qf[GM][KC][X];
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      const T* qrow = static_cast<const T*>(a.q) +
                      (static_cast<int64_t>(s) * a.n_q_heads + kvh * G + (gi < G ? gi : 0)) * D;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        T tmp[X];
        const uint4 bits = *reinterpret_cast<const uint4*>(qrow + (4 * kc + g) * X);
        __builtin_memcpy(tmp, &bits, 16);
#pragma unroll
        for (int e = 0; e < X; ++e) qf[gi][kc][e] = to_f32(tmp[e]);
      }
    }

    float m_run[GM], l_part[GM], acc[RPL][GM];
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      m_run[gi] = -INFINITY;
      l_part[gi] = 0.f;
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr) acc[rr][gi] = 0.f;
    }

    for (int w0 = 0; w0 < nblk; w0 += 64) {
      const int wb = min(64, nblk - w0);
      int bid = lane < wb ? bt[w0 + lane] : 0;
      bid = min(max(bid, 0), a.num_blocks - 1);
      const int wend = min(ntok, (w0 + 64) << lb);
      for (int t0 = w0 << lb; t0 < wend; t0 += 16) {
        // keys: lane (token r16, column group g)
        const int j = t0 + r16;
        uint4 kf[KC];
        {
          const int b = lane_fetch(bid, (j >> lb) - w0);
          const T* kb = kbase + static_cast<int64_t>(b) * blk_stride + (j & (Bsz - 1)) * X;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc)
            kf[kc] = *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(4 * kc + g) * Bsz * X);
        }
        // values: lane (row vrow + RSTEP*rr, tokens t0 + vpart*X .. +X-1)
        uint4 vv[RPL];
        const int jv = t0 + vpart * X;
        {
          const int b = lane_fetch(bid, (jv >> lb) - w0);
          const T* vb = vbase + static_cast<int64_t>(b) * blk_stride + (jv & (Bsz - 1));
#pragma unroll
          for (int rr = 0; rr < RPL; ++rr)
            vv[rr] = *reinterpret_cast<const uint4*>(vb + static_cast<int64_t>(vrow + RSTEP * rr) * Bsz);
        }
        const bool partial = t0 + 16 > ntok;
        float p[GM];
#pragma unroll
        for (int gi = 0; gi < GM; ++gi) {
          float dot = 0.f;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            T tmp[X];
            __builtin_memcpy(tmp, &kf[kc], 16);
#pragma unroll
            for (int e = 0; e < X; ++e) dot = fmaf(qf[gi][kc][e], to_f32(tmp[e]), dot);
          }
          dot += xor_f(dot, 16);
          dot += xor_f(dot, 32);
          float xs = dot * a.scale_log2;
          if (partial && j >= ntok) xs = -INFINITY;
          float mt = xs;
          mt = fmaxf(mt, xor_f(mt, 1));
          mt = fmaxf(mt, xor_f(mt, 2));
          mt = fmaxf(mt, xor_f(mt, 4));
          mt = fmaxf(mt, xor_f(mt, 8));
          const float m_new = fmaxf(m_run[gi], mt);
          const float alpha = fast_exp2(m_run[gi] - m_new);
          m_run[gi] = m_new;
          p[gi] = fast_exp2(xs - m_new);
          l_part[gi] = l_part[gi] * alpha + (g == 0 ? p[gi] : 0.f);
#pragma unroll
          for (int rr = 0; rr < RPL; ++rr) acc[rr][gi] *= alpha;
        }
        // weighted values
#pragma unroll
        for (int e = 0; e < X; ++e) {
          const bool tok_ok = !partial || (jv + e < ntok);
          float pe[GM];
#pragma unroll
          for (int gi = 0; gi < GM; ++gi) pe[gi] = lane_fetch(p[gi], vpart * X + e);
#pragma unroll
          for (int rr = 0; rr < RPL; ++rr) {
            T tmp[X];
            __builtin_memcpy(tmp, &vv[rr], 16);
            const float vval = tok_ok ? to_f32(tmp[e]) : 0.f;
#pragma unroll
            for (int gi = 0; gi < GM; ++gi) acc[rr][gi] = fmaf(pe[gi], vval, acc[rr][gi]);
          }
        }
      }
    }

    // ---- finish
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      float lt = l_part[gi];
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) lt += xor_f(lt, m);
      l_part[gi] = lt;
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr) {
#pragma unroll
        for (int m = 1; m < PPR; m <<= 1) acc[rr][gi] += xor_f(acc[rr][gi], m);
      }
    }
    if (vpart == 0) {
#pragma unroll
      for (int gi = 0; gi < GM; ++gi) {
        if (gi >= G) break;
        const int64_t row = static_cast<int64_t>(s) * a.n_q_heads + kvh * G + gi;
        if (nparts == 1) {
          const float inv = 1.f / l_part[gi];
#pragma unroll
          for (int rr = 0; rr < RPL; ++rr)
            store1<T>(a.out, row * D + vrow + RSTEP * rr, acc[rr][gi] * inv, a.out_f32);
        } else {
          const int64_t pidx = row * a.max_parts + part;
#pragma unroll
          for (int rr = 0; rr < RPL; ++rr) a.part_acc[pidx * D + vrow + RSTEP * rr] = acc[rr][gi];
          if (lane == 0) {
            a.part_m[pidx] = m_run[gi];
            a.part_l[pidx] = l_part[gi];
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------ merge
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p with M = max_p m_p, for rows with more
// than one partition.  One workgroup per (row, head): its 4 waves take every 4th partition and
// keep a running (max, numerator, denominator) with rescaling, so each wave's loads are
// independent and pipeline; the 4 running states are combined through LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;  // output elements per lane
  const int s = blockIdx.x;
  const int head = blockIdx.y;
  const int L = row_len(a, s);
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t pbase = (static_cast<int64_t>(s) * a.n_q_heads + head) * a.max_parts;
  float M = -INFINITY, den = 0.f, num[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) num[i] = 0.f;
#pragma unroll 4
  for (int p = wave; p < np; p += 4) {
    const float m = a.part_m[pbase + p];
    const float l = a.part_l[pbase + p];
    float v[PER];
    if constexpr (PER == 2) {
      const float2 t = *reinterpret_cast<const float2*>(a.part_acc + (pbase + p) * D + 2 * lane);
      v[0] = t.x;
      v[1] = t.y;
    } else {
      v[0] = a.part_acc[(pbase + p) * D + lane];
    }
    const float Mn = fmaxf(M, m);
    const float so = fast_exp2(M - Mn), sn = fast_exp2(m - Mn);
#pragma unroll
    for (int i = 0; i < PER; ++i) num[i] = num[i] * so + v[i] * sn;
    den = den * so + l * sn;
    M = Mn;
  }
  __shared__ float sM[4], sden[4], snum[4][D];
  if (lane == 0) {
    sM[wave] = M;
    sden[wave] = den;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) snum[wave][PER * lane + i] = num[i];
  __syncthreads();
  if (wave != 0) return;
  const float Mt = fmaxf(fmaxf(sM[0], sM[1]), fmaxf(sM[2], sM[3]));
  float dt = 0.f, nt[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) nt[i] = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float sc = fast_exp2(sM[w] - Mt);   // 0 for a wave that saw no partition
    dt += sden[w] * sc;
#pragma unroll
    for (int i = 0; i < PER; ++i) nt[i] += snum[w][PER * lane + i] * sc;
  }
  const float inv = 1.f / dt;
  const int64_t row = static_cast<int64_t>(s) * a.n_q_heads + head;
#pragma unroll
  for (int i = 0; i < PER; ++i) store1<T>(a.out, row * D + PER * lane + i, nt[i] * inv, a.out_f32);
}

// ------------------------------------------------------------------------------ dispatch
template <typename T, int D>
const void* mfma_kernel_ptr_d(int block_size) {
  switch (block_size) {
    case 8: return reinterpret_cast<const void*>(&decode_mfma_kernel<T, D, 8>);
    case 16: return reinterpret_cast<const void*>(&decode_mfma_kernel<T, D, 16>);
    case 32: return reinterpret_cast<const void*>(&decode_mfma_kernel<T, D, 32>);
    default: return nullptr;
  }
}
template <typename T>
const void* mfma_kernel_ptr(int head_dim, int block_size) {
  return head_dim == 128 ? mfma_kernel_ptr_d<T, 128>(block_size) : mfma_kernel_ptr_d<T, 64>(block_size);
}

template <typename T>
hipError_t main_dispatch(const DecodeArgs& a, int head_dim, int path, int32_t grid, hipStream_t st) {
  const dim3 blk(64), grd(grid);
  if (path == 1) {
    if constexpr (sizeof(T) == 2) {
      const void* fn = mfma_kernel_ptr<T>(head_dim, a.block_size);
      if (!fn) return hipErrorInvalidValue;
      void* args[] = {const_cast<DecodeArgs*>(&a)};
      return hipLaunchKernel(fn, grd, blk, args, 0, st);
    }
    return hipErrorInvalidValue;
  }
  const bool one = a.group == 1;
  if (head_dim == 128) {
    if (one) decode_vec_kernel<T, 128, 1><<<grd, blk, 0, st>>>(a);
    else decode_vec_kernel<T, 128, 4><<<grd, blk, 0, st>>>(a);
  } else {
    if (one) decode_vec_kernel<T, 64, 1><<<grd, blk, 0, st>>>(a);
    else decode_vec_kernel<T, 64, 4><<<grd, blk, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <typename T>
const void* main_kernel_ptr(int head_dim, int path, int group, int block_size) {
  if (path == 1) {
    if constexpr (sizeof(T) == 2) return mfma_kernel_ptr<T>(head_dim, block_size);
    return nullptr;
  }
  if (head_dim == 128)
    return group == 1 ? reinterpret_cast<const void*>(&decode_vec_kernel<T, 128, 1>)
                      : reinterpret_cast<const void*>(&decode_vec_kernel<T, 128, 4>);
  return group == 1 ? reinterpret_cast<const void*>(&decode_vec_kernel<T, 64, 1>)
                    : reinterpret_cast<const void*>(&decode_vec_kernel<T, 64, 4>);
}

}  // namespace

hipError_t launch_decode_plan(const DecodeArgs& a, int dtype, int head_dim, hipStream_t st) {
  if (dtype == PKV_F32) decode_plan_kernel<float><<<1, 1024, 0, st>>>(a, head_dim);
  else if (dtype == PKV_F16) decode_plan_kernel<_Float16><<<1, 1024, 0, st>>>(a, head_dim);
  else decode_plan_kernel<__bf16><<<1, 1024, 0, st>>>(a, head_dim);
  return hipGetLastError();
}

hipError_t launch_decode_main(const DecodeArgs& a, int dtype, int head_dim, int path, int32_t grid,
                              hipStream_t st) {
  if (dtype == PKV_F32) return main_dispatch<float>(a, head_dim, path, grid, st);
  if (dtype == PKV_F16) return main_dispatch<_Float16>(a, head_dim, path, grid, st);
  return main_dispatch<__bf16>(a, head_dim, path, grid, st);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim, hipStream_t st) {
  const dim3 grd(a.num_seqs, a.n_q_heads), blk(256);
  if (dtype == PKV_F32) {
    if (head_dim == 128) decode_reduce_kernel<float, 128><<<grd, blk, 0, st>>>(a);
    else decode_reduce_kernel<float, 64><<<grd, blk, 0, st>>>(a);
  } else if (dtype == PKV_F16) {
    if (head_dim == 128) decode_reduce_kernel<_Float16, 128><<<grd, blk, 0, st>>>(a);
    else decode_reduce_kernel<_Float16, 64><<<grd, blk, 0, st>>>(a);
  } else {
    if (head_dim == 128) decode_reduce_kernel<__bf16, 128><<<grd, blk, 0, st>>>(a);
    else decode_reduce_kernel<__bf16, 64><<<grd, blk, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t decode_main_grid_cap(int dtype, int head_dim, int path, int group, int block_size, int32_t* cap) {
  const void* fn = dtype == PKV_F32   ? main_kernel_ptr<float>(head_dim, path, group, block_size)
                   : dtype == PKV_F16 ? main_kernel_ptr<_Float16>(head_dim, path, group, block_size)
                                      : main_kernel_ptr<__bf16>(head_dim, path, group, block_size);
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
