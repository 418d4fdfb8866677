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

__device__ inline int row_len(const DecodeArgs& a, int s) {
  const int L = a.seq_lens[s];
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
template <typename T>
__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a, int head_dim) {
  __shared__ int sums[1024];
  const int S = a.num_seqs;
  const int tid = threadIdx.x;
  const int per = (S + 1023) / 1024;
  const int lo = min(S, tid * per);
  const int hi = min(S, lo + per);
  int local = 0;
  for (int s = lo; s < hi; ++s) {
    const int L = row_len(a, s);
    local += (L + a.part_tokens - 1) / a.part_tokens;
  }
  sums[tid] = local;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? sums[tid - d] : 0;
    __syncthreads();
    sums[tid] += v;
    __syncthreads();
  }
  int off = sums[tid] - local;
  const int64_t row_elems = static_cast<int64_t>(a.n_q_heads) * head_dim;
  for (int s = lo; s < hi; ++s) {
    const int L = row_len(a, s);
    const int np = (L + a.part_tokens - 1) / a.part_tokens;
    for (int p = 0; p < np; ++p) a.units[off + p] = make_int2(s, p);
    off += np;
    if (L == 0) {  // empty row: zeros
      for (int64_t i = 0; i < row_elems; ++i) store1<T>(a.out, s * row_elems + i, 0.f, a.out_f32);
    }
  }
  if (tid == 1023) {
    a.counters[0] = sums[1023];
    a.counters[1] = 0;
  }
}

// ------------------------------------------------------------------------------ MFMA path
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_mfma_kernel(DecodeArgs a) {
  using V8 = typename Vec8<T>::type;
  constexpr int X = 8;        // 16-bit elements per 16-byte vector
  constexpr int KS = D / 32;  // MFMA k-steps over head_dim
  constexpr int DT = D / 16;  // 16-row tiles of head_dim in PV
  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int g = lane >> 4;
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
    const int head = kvh * G + r16;
    const bool hvalid = r16 < G;
    const T* kbase = kpool + static_cast<int64_t>(kvh) * chunk;
    const T* vbase = vpool + static_cast<int64_t>(kvh) * chunk;

    // q^T as the B operand of S^T = K q^T: lane (g, h) holds q[h][8*(4ks+g) .. +8].
    V8 qf[KS];
    {
      const T* qrow = static_cast<const T*>(a.q) + (static_cast<int64_t>(s) * a.n_q_heads + head) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 bits = make_uint4(0, 0, 0, 0);
        if (hvalid) bits = *reinterpret_cast<const uint4*>(qrow + 8 * (4 * ks + g));
        __builtin_memcpy(&qf[ks], &bits, 16);
      }
    }

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int w0 = 0; w0 < nblk; w0 += 64) {
      const int wb = min(64, nblk - w0);
      int bid = lane < wb ? bt[w0 + lane] : 0;
      bid = min(max(bid, 0), a.num_blocks - 1);
      const int wend = min(ntok, (w0 + 64) << lb);
      for (int t0 = w0 << lb; t0 < wend; t0 += 32) {
        // ---- loads: key rows (two halves of 16 tokens), value columns
        uint4 kf[2][KS];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j = t0 + 16 * hf + r16;
          const int b = lane_fetch(bid, (j >> lb) - w0);
          const T* kb = kbase + static_cast<int64_t>(b) * blk_stride + (j & (Bsz - 1)) * X;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            kf[hf][ks] = *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(4 * ks + g) * Bsz * X);
        }
        uint2 vf[DT][2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j = t0 + 16 * hf + 4 * g;
          const int b = lane_fetch(bid, (j >> lb) - w0);
          const T* vb = vbase + static_cast<int64_t>(b) * blk_stride + (j & (Bsz - 1));
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            vf[dt][hf] = *reinterpret_cast<const uint2*>(vb + static_cast<int64_t>(16 * dt + r16) * Bsz);
        }
        // ---- S^T[token][head] for the two halves
        float x[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            V8 kv;
            __builtin_memcpy(&kv, &kf[hf][ks], 16);
            sc = mfma_16x16x32(kv, qf[ks], sc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) x[4 * hf + i] = sc[i] * a.scale_log2;
        }
        const bool partial = t0 + 32 > ntok;
        if (partial) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (t0 + 16 * (e >> 2) + 4 * g + (e & 3) >= ntok) x[e] = -INFINITY;
        }
        // ---- online softmax (base 2)
        float mt = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, x[e]);
        mt = fmaxf(mt, xor_f(mt, 16));
        mt = fmaxf(mt, xor_f(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        V8 pv;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const T pt = static_cast<T>(fast_exp2(x[e] - m_new));
          pv[e] = pt;
          psum += to_f32(pt);
        }
        l_run = l_run * alpha + psum;
        // ---- O^T[dim][head] += V^T P^T
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          V8 va;
          __builtin_memcpy(&va, &vf[dt][0], 8);
          __builtin_memcpy(reinterpret_cast<char*>(&va) + 8, &vf[dt][1], 8);
          if (partial) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (t0 + 16 * (e >> 2) + 4 * g + (e & 3) >= ntok) va[e] = static_cast<T>(0.f);
          }
          acc[dt] = mfma_16x16x32(va, pv, acc[dt] * alpha);
        }
      }
    }

    // ---- finish: total weight per head, then output or partial
    float l_tot = l_run + xor_f(l_run, 16);
    l_tot += xor_f(l_tot, 32);
    if (hvalid) {
      const int64_t row = static_cast<int64_t>(s) * a.n_q_heads + head;
      if (nparts == 1) {
        const float inv = 1.f / l_tot;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) store4<T>(a.out, row * D + 16 * dt + 4 * g, acc[dt] * inv, a.out_f32);
      } else {
        const int64_t pidx = row * a.max_parts + part;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<f32x4*>(a.part_acc + pidx * D + 16 * dt + 4 * g) = acc[dt];
        if (g == 0) {
          a.part_m[pidx] = m_run;
          a.part_l[pidx] = l_tot;
        }
      }
    }
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
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, M = max_p m_p, for rows with
// more than one partition.  Block (s, y): 4 waves split the partitions of 64
// (head, 4-dim) outputs and combine through LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int D4 = D / 4;
  const int s = blockIdx.x;
  const int L = row_len(a, s);
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.y * 64 + lane;
  const int head = idx / D4;
  const int d4 = idx - head * D4;
  const bool valid = head < a.n_q_heads;
  const int64_t pbase = (static_cast<int64_t>(s) * a.n_q_heads + (valid ? head : 0)) * a.max_parts;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_m[pbase + p]);
  f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (valid) {
    for (int p = wave; p < np; p += 4) {
      const float w = fast_exp2(a.part_m[pbase + p] - M);
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.part_acc + (pbase + p) * D + 4 * d4);
      num += w * v;
      den += w * a.part_l[pbase + p];
    }
  }
  __shared__ f32x4 snum[3][64];
  __shared__ float sden[3][64];
  if (wave > 0) {
    snum[wave - 1][lane] = num;
    sden[wave - 1][lane] = den;
  }
  __syncthreads();
  if (wave == 0 && valid) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      num += snum[w][lane];
      den += sden[w][lane];
    }
    const int64_t row = static_cast<int64_t>(s) * a.n_q_heads + head;
    store4<T>(a.out, row * D + 4 * d4, num * (1.f / den), a.out_f32);
  }
}

// ------------------------------------------------------------------------------ dispatch
template <typename T>
hipError_t main_dispatch(const DecodeArgs& a, int head_dim, int path, int32_t grid, hipStream_t st) {
  const dim3 blk(64), grd(grid);
  if (path == 1) {
    if constexpr (sizeof(T) == 2) {
      if (head_dim == 128) decode_mfma_kernel<T, 128><<<grd, blk, 0, st>>>(a);
      else decode_mfma_kernel<T, 64><<<grd, blk, 0, st>>>(a);
      return hipGetLastError();
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
const void* main_kernel_ptr(int head_dim, int path, int group) {
  if (path == 1) {
    if constexpr (sizeof(T) == 2) {
      return head_dim == 128 ? reinterpret_cast<const void*>(&decode_mfma_kernel<T, 128>)
                             : reinterpret_cast<const void*>(&decode_mfma_kernel<T, 64>);
    }
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
  const dim3 grd(a.num_seqs, (a.n_q_heads * (head_dim / 4) + 63) / 64), blk(256);
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

hipError_t decode_main_grid_cap(int dtype, int head_dim, int path, int group, int32_t* cap) {
  const void* fn = dtype == PKV_F32   ? main_kernel_ptr<float>(head_dim, path, group)
                   : dtype == PKV_F16 ? main_kernel_ptr<_Float16>(head_dim, path, group)
                                      : main_kernel_ptr<__bf16>(head_dim, path, group);
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
