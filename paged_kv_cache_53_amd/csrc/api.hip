// C-ABI entry points of libpagedkv: argument checks, workspace carve-up, kernel dispatch,
// and the optional per-kernel event timing.  Every check runs before anything is launched.
#include <cmath>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace pkv {

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline int esize(int dtype) { return dtype == PKV_F32 ? 4 : dtype == PKV_FP8_E4M3 ? 1 : 2; }
// element types of rows, q and results
inline bool valid_dtype(int d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }
// element types a pool may hold
inline bool valid_pool_dtype(int d) { return valid_dtype(d) || d == PKV_FP8_E4M3; }
inline bool valid_scale(float s) { return s > 0.f && s <= 3.402823466e38f; }   // positive, finite
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int log2i(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// ---- kernel timing -----------------------------------------------------------------
struct TimingRecord {
  int kernel;
  hipEvent_t start, stop;
};

struct Timing {
  std::mutex mu;
  bool enabled = false;
  uint32_t mask = ~0u;   // kernel ids timed while enabled
  std::vector<TimingRecord> pending;
  std::vector<hipEvent_t> spare;
  hipEvent_t open_start = nullptr;  // recorded by timing_before, closed by timing_after
  int open_kernel = -1;

  hipEvent_t take() {
    if (!spare.empty()) {
      hipEvent_t e = spare.back();
      spare.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void give(hipEvent_t e) {
    if (e) spare.push_back(e);
  }
  void drop_pending() {
    for (auto& r : pending) {
      give(r.start);
      give(r.stop);
    }
    pending.clear();
    give(open_start);
    open_start = nullptr;
  }
};

Timing& timing() {
  static Timing* t = new Timing();  // lives until process exit; events are never destroyed
  return *t;
}

// ---- persistent-grid cap cache per (device, kernel variant) ---------------------------
std::mutex cap_mu;
std::unordered_map<int64_t, int32_t> cap_cache;

hipError_t grid_cap(int dtype, bool kv_fp8, bool flat, int head_dim, int path, int group, int block_size,
                    int pol, int32_t* cap) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  // one entry per kernel variant: the vector path has one variant per group width (1, 2, 3-4),
  // the MFMA path one per storage type and one for flat spans, each for every load policy
  const int variant = path == 1 ? (flat ? 5 : kv_fp8 ? 4 : 3) : (group == 1 ? 0 : group == 2 ? 1 : 2);
  const int64_t key = (((((static_cast<int64_t>(dev) * 4 + dtype) * 512 + head_dim) * 8 + variant) * 64) +
                       block_size) * 4 + pol;
  {
    std::lock_guard<std::mutex> g(cap_mu);
    auto it = cap_cache.find(key);
    if (it != cap_cache.end()) {
      *cap = it->second;
      return hipSuccess;
    }
  }
  e = decode_main_grid_cap(dtype, kv_fp8, flat, head_dim, path, group, block_size, pol, cap);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(cap_mu);
  cap_cache[key] = *cap;
  return hipSuccess;
}

}  // namespace

void timing_before(int kernel, hipStream_t stream) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.enabled || !((t.mask >> kernel) & 1u)) return;
  t.give(t.open_start);
  t.open_start = t.take();
  t.open_kernel = kernel;
  if (t.open_start && hipEventRecord(t.open_start, stream) != hipSuccess) {
    t.give(t.open_start);
    t.open_start = nullptr;
  }
}

void timing_after(int kernel, hipStream_t stream) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.enabled || !t.open_start || t.open_kernel != kernel) return;
  hipEvent_t stop = t.take();
  if (stop && hipEventRecord(stop, stream) == hipSuccess) {
    t.pending.push_back({kernel, t.open_start, stop});
  } else {
    t.give(t.open_start);
    t.give(stop);
  }
  t.open_start = nullptr;
}

int32_t partition_tokens(int32_t max_seq_len, int32_t partition_size) {
  if (partition_size > 0) return partition_size;
  const int32_t L = max_seq_len > 0 ? max_seq_len : 1;
  return (L + 31) / 32 * 32;
}

WorkspaceLayout workspace_layout(int32_t num_seqs, int32_t n_q_heads, int32_t head_dim, int32_t max_parts) {
  WorkspaceLayout w{};
  const size_t units = static_cast<size_t>(num_seqs) * max_parts;
  const size_t parts = units * n_q_heads;
  w.counters_off = 0;
  w.units_off = 256;
  w.m_off = round_up(w.units_off + units * sizeof(int4), 256);
  w.l_off = round_up(w.m_off + parts * sizeof(float), 256);
  w.acc_off = round_up(w.l_off + parts * sizeof(float), 256);
  w.total = round_up(w.acc_off + parts * head_dim * sizeof(float), 256);
  return w;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_OOM: return "out of KV-cache blocks";
    case PKV_ERR_NOT_FOUND: return "unknown sequence";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or type";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_SCRATCH: return "needs more than the library's static scratch (PKV_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int pkv_version(void) { return 2; }

size_t pkv_pool_bytes(int32_t num_blocks, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                      int dtype) {
  if (num_blocks <= 0 || n_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || !valid_pool_dtype(dtype))
    return 0;
  const int X = 16 / esize(dtype);
  if (head_dim % X) return 0;
  return static_cast<size_t>(num_blocks) * n_kv_heads * head_dim * block_size * esize(dtype);
}

int pkv_reshape_and_cache(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                          int64_t k_token_stride, int64_t v_token_stride, void* k_pool, void* v_pool,
                          int32_t num_blocks, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                          int dtype, void* stream) {
  if (num_tokens < 0 || !valid_dtype(dtype) || num_blocks <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0)
    return PKV_ERR_INVALID;
  const int es = esize(dtype);
  const int X = 16 / es;
  if (head_dim % X) return PKV_ERR_INVALID;
  const int64_t row = static_cast<int64_t>(n_kv_heads) * head_dim;
  const int64_t ks = k_token_stride == 0 ? row : k_token_stride;
  const int64_t vs = v_token_stride == 0 ? row : v_token_stride;
  if (ks < row || vs < row || (ks * es) % 16 || (vs * es) % 16) return PKV_ERR_INVALID;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PKV_ERR_INVALID;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(slot_mapping, 8))
    return PKV_ERR_INVALID;
  ScatterArgs a{k, v, slot_mapping, k_pool, v_pool, ks, vs, num_tokens, num_blocks, n_kv_heads,
                head_dim, block_size};
  hipStream_t st = static_cast<hipStream_t>(stream);
  timing_before(PKV_K_RESHAPE_AND_CACHE, st);
  const hipError_t e = launch_reshape_and_cache(a, dtype, st);
  timing_after(PKV_K_RESHAPE_AND_CACHE, st);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_reshape_and_cache_fp8(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                              int64_t k_token_stride, int64_t v_token_stride, void* k_pool, void* v_pool,
                              int32_t num_blocks, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                              int src_dtype, float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0 || !valid_dtype(src_dtype) || num_blocks <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || !valid_scale(k_scale) || !valid_scale(v_scale))
    return PKV_ERR_INVALID;
  const int es = esize(src_dtype);
  if (head_dim % 16) return PKV_ERR_INVALID;   // 16 codes per key vector
  const int64_t row = static_cast<int64_t>(n_kv_heads) * head_dim;
  const int64_t ks = k_token_stride == 0 ? row : k_token_stride;
  const int64_t vs = v_token_stride == 0 ? row : v_token_stride;
  if (ks < row || vs < row || (ks * es) % 16 || (vs * es) % 16) return PKV_ERR_INVALID;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PKV_ERR_INVALID;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(slot_mapping, 8))
    return PKV_ERR_INVALID;
  ScatterArgs a{k, v, slot_mapping, k_pool, v_pool, ks, vs, num_tokens, num_blocks, n_kv_heads,
                head_dim, block_size};
  hipStream_t st = static_cast<hipStream_t>(stream);
  timing_before(PKV_K_RESHAPE_AND_CACHE, st);
  const hipError_t e = launch_reshape_and_cache_fp8(a, src_dtype, k_scale, v_scale, st);
  timing_after(PKV_K_RESHAPE_AND_CACHE, st);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n_pairs, int32_t num_blocks,
                    int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int dtype, void* stream) {
  if (n_pairs < 0 || !valid_pool_dtype(dtype) || num_blocks <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0)
    return PKV_ERR_INVALID;
  const int64_t block_bytes = static_cast<int64_t>(n_kv_heads) * head_dim * block_size * esize(dtype);
  if (block_bytes % 16) return PKV_ERR_UNSUPPORTED;
  if (n_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !pairs) return PKV_ERR_INVALID;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(pairs, 4)) return PKV_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  timing_before(PKV_K_COPY_BLOCKS, st);
  const hipError_t e = launch_copy_blocks(k_pool, v_pool, pairs, n_pairs, num_blocks, block_bytes, st);
  timing_after(PKV_K_COPY_BLOCKS, st);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"

namespace {

// The address a kernel uses for p: device memory as is, pinned (registered) host memory through its
// device mapping.  Anything else (pageable host memory, a bad pointer) is rejected before a launch.
bool kernel_address(const void* p, const void** out) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error the query may leave
    return false;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *out = p;
    return true;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer) {
    // the mapping of the allocation's base, offset to p
    const char* host_base = static_cast<const char*>(at.hostPointer);
    *out = static_cast<const char*>(at.devicePointer) + (static_cast<const char*>(p) - host_base);
    return true;
  }
  return false;
}

}  // namespace

extern "C" {

int pkv_swap_blocks(const void* src_k, const void* src_v, int32_t src_blocks, void* dst_k, void* dst_v,
                    int32_t dst_blocks, const int32_t* pairs, int32_t n_pairs, int32_t n_kv_heads,
                    int32_t head_dim, int32_t block_size, int dtype, void* stream) {
  if (n_pairs < 0 || src_blocks <= 0 || dst_blocks <= 0 || !valid_pool_dtype(dtype) || n_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0)
    return PKV_ERR_INVALID;
  const int64_t block_bytes = static_cast<int64_t>(n_kv_heads) * head_dim * block_size * esize(dtype);
  if (block_bytes % 16) return PKV_ERR_UNSUPPORTED;
  if (n_pairs == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PKV_ERR_INVALID;
  if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 16) || !aligned(dst_v, 16) || !aligned(pairs, 4))
    return PKV_ERR_INVALID;
  const void *sk, *sv, *dk, *dv, *pp;
  if (!kernel_address(src_k, &sk) || !kernel_address(src_v, &sv) || !kernel_address(dst_k, &dk) ||
      !kernel_address(dst_v, &dv) || !kernel_address(pairs, &pp))
    return PKV_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  timing_before(PKV_K_SWAP_BLOCKS, st);
  const hipError_t e = launch_move_blocks(sk, sv, src_blocks, const_cast<void*>(dk), const_cast<void*>(dv),
                                          dst_blocks, static_cast<const int32_t*>(pp), n_pairs, block_bytes, st);
  timing_after(PKV_K_SWAP_BLOCKS, st);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_append_slots(const int64_t* slot_mapping, int32_t num_seqs, int32_t* block_tables,
                     int32_t block_table_stride, int32_t* seq_lens, int32_t block_size, void* stream) {
  if (num_seqs < 0 || block_table_stride <= 0 || block_size <= 0) return PKV_ERR_INVALID;
  if (num_seqs == 0) return PKV_OK;
  if (!slot_mapping || !block_tables || !seq_lens) return PKV_ERR_INVALID;
  if (!aligned(slot_mapping, 8) || !aligned(block_tables, 4) || !aligned(seq_lens, 4)) return PKV_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  timing_before(PKV_K_APPEND_SLOTS, st);
  const hipError_t e = launch_append_slots(slot_mapping, num_seqs, block_tables, block_table_stride,
                                           seq_lens, block_size, st);
  timing_after(PKV_K_APPEND_SLOTS, st);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t pkv_paged_attention_workspace_size(int32_t num_seqs, int32_t n_q_heads, int32_t head_dim,
                                          int32_t max_seq_len, int32_t partition_size) {
  if (num_seqs < 0 || n_q_heads <= 0 || head_dim <= 0 || max_seq_len < 0 || partition_size < 0 ||
      (partition_size % 32))
    return 0;
  const int32_t P = partition_tokens(max_seq_len, partition_size);
  const int32_t max_parts = max_seq_len > 0 ? (max_seq_len + P - 1) / P : 1;
  return workspace_layout(num_seqs, n_q_heads, head_dim, max_parts).total;
}

int pkv_paged_attention_decode(void* out, int out_dtype, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_tables, int32_t block_table_stride,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, float scale, int32_t max_seq_len, int32_t partition_size,
                               void* workspace, size_t workspace_bytes, int kv_dtype, void* stream) {
  return pkv_paged_attention_decode_ex(out, out_dtype, q, k_pool, v_pool, block_tables, block_table_stride,
                                       seq_lens, num_seqs, n_q_heads, n_kv_heads, head_dim, block_size,
                                       num_blocks, scale, max_seq_len, partition_size, workspace,
                                       workspace_bytes, kv_dtype, 0u, stream);
}

}  // extern "C"

namespace {

// A checked decode call, ready to launch.
struct DecodeLaunch {
  DecodeArgs a;
  int kv_dtype, head_dim, path, pol;
  bool kv_fp8;
  int32_t grid;
  bool empty;   // no rows: nothing to launch
};

// Every check of a decode call, then its kernel arguments.  q_dtype: the type of q (and of out
// unless out is fp32); kv_fp8: the pools hold E4M3 codes with scales k_scale / v_scale (else they
// hold q_dtype); flat_bps > 0: flat spans of flat_bps blocks, block_tables then holds one span
// index per row.
int decode_prepare(DecodeLaunch* L, void* out, int out_dtype, const void* q, int q_dtype, const void* k_pool,
                   const void* v_pool, bool kv_fp8, float k_scale, float v_scale, const int32_t* block_tables,
                   int32_t block_table_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t n_q_heads,
                   int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                   int32_t max_seq_len, int32_t partition_size, void* workspace, size_t workspace_bytes,
                   uint32_t flags, int32_t flat_bps = 0, int32_t shared_prefix_tokens = 0) {
  L->empty = false;
  if (shared_prefix_tokens < 0) return PKV_ERR_INVALID;
  const int kv_dtype = q_dtype;   // the compute type of the kernels
  const bool flat = flat_bps > 0;
  if (flags & ~static_cast<uint32_t>(PKV_DECODE_SHARED_KV | PKV_DECODE_VECTOR)) return PKV_ERR_INVALID;
  // ---- shape and type checks
  if (!valid_dtype(kv_dtype) || !(out_dtype == kv_dtype || out_dtype == PKV_F32)) return PKV_ERR_INVALID;
  if (kv_fp8 && (!valid_scale(k_scale) || !valid_scale(v_scale))) return PKV_ERR_INVALID;
  if (num_seqs < 0 || n_q_heads <= 0 || n_q_heads > 65535 || n_kv_heads <= 0 || (n_q_heads % n_kv_heads) ||
      num_blocks <= 0 ||
      max_seq_len < 0 || partition_size < 0 || (partition_size % 32) || block_size <= 0 ||
      !std::isfinite(scale))
    return PKV_ERR_INVALID;
  if (block_size != 8 && block_size != 16 && block_size != 32) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  const int group = n_q_heads / n_kv_heads;
  int path;
  if (kv_dtype == PKV_F32) {
    if (kv_fp8 || group > 4) return PKV_ERR_UNSUPPORTED;   // a quantised cache takes bf16 or f16 q
    path = 0;
  } else {
    if (group > 16) return PKV_ERR_UNSUPPORTED;
    path = 1;   // MFMA for every group size (heads padded to 16)
    if (flags & PKV_DECODE_VECTOR) {   // per-token dot products and shuffle reductions instead
      if (kv_fp8 || group > 1) return PKV_ERR_UNSUPPORTED;
      path = 0;
    }
  }
  const int64_t max_blocks = (static_cast<int64_t>(max_seq_len) + block_size - 1) / block_size;
  if (flat) {
    if (kv_fp8 || kv_dtype == PKV_F32) return PKV_ERR_UNSUPPORTED;   // flat spans: 16-bit KV
    if (max_blocks > flat_bps || num_blocks % flat_bps) return PKV_ERR_INVALID;
    if (flags & PKV_DECODE_SHARED_KV) return PKV_ERR_UNSUPPORTED;    // spans are never shared
    if (path != 1) return PKV_ERR_UNSUPPORTED;                        // spans decode on MFMA
  } else if (block_table_stride < max_blocks || block_table_stride < 0) {
    return PKV_ERR_INVALID;
  }
  const int32_t P = partition_tokens(max_seq_len, partition_size);
  const int32_t max_parts = max_seq_len > 0 ? (max_seq_len + P - 1) / P : 1;
  const int64_t unit_bound = static_cast<int64_t>(num_seqs) * max_parts * n_kv_heads;
  if (unit_bound >= (int64_t{1} << 31)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) {
    L->empty = true;
    return PKV_OK;
  }
  // ---- pointer checks
  if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens || !workspace) return PKV_ERR_INVALID;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(workspace, 256))
    return PKV_ERR_INVALID;
  const WorkspaceLayout wl = workspace_layout(num_seqs, n_q_heads, head_dim, max_parts);
  if (workspace_bytes < wl.total) return PKV_ERR_INVALID;

  char* ws = static_cast<char*>(workspace);
  DecodeArgs& a = L->a;
  a = DecodeArgs{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.counters = reinterpret_cast<int32_t*>(ws + wl.counters_off);
  a.units = reinterpret_cast<int4*>(ws + wl.units_off);
  a.part_m = reinterpret_cast<float*>(ws + wl.m_off);
  a.part_l = reinterpret_cast<float*>(ws + wl.l_off);
  a.part_acc = reinterpret_cast<float*>(ws + wl.acc_off);
  a.bt_stride = block_table_stride;
  a.num_seqs = num_seqs;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.log2_block = log2i(block_size);
  a.max_seq_len = max_seq_len;
  a.part_tokens = P;
  a.max_parts = max_parts;
  a.out_f32 = out_dtype == PKV_F32 ? 1 : 0;
  a.scale_log2 = (kv_fp8 ? scale * k_scale : scale) * 1.4426950408889634f;
  a.v_scale = kv_fp8 ? v_scale : 1.f;
  a.flat_bps = flat ? flat_bps : 0;

  // load policy: tiles in the rows' shared prefix cacheable and the rest streamed (MFMA path), else
  // everything cacheable when blocks are shared, else everything streamed
  int pol = (flags & PKV_DECODE_SHARED_KV) ? kLoadCached : kLoadStreamed;
  if (shared_prefix_tokens > 0) {
    if (flat) return PKV_ERR_UNSUPPORTED;   // spans are never shared
    pol = path == 1 ? kLoadMixed : kLoadCached;
  }
  a.cache_tokens = pol == kLoadMixed ? shared_prefix_tokens : 0;
  int32_t cap = 0;
  if (grid_cap(kv_dtype, kv_fp8, flat, head_dim, path, group, block_size, pol, &cap) != hipSuccess) return PKV_ERR_HIP;
  L->grid = static_cast<int32_t>(unit_bound < cap ? (unit_bound > 0 ? unit_bound : 1) : cap);
  L->kv_dtype = kv_dtype;
  L->head_dim = head_dim;
  L->path = path;
  L->kv_fp8 = kv_fp8;
  L->pol = pol;
  return PKV_OK;
}

// The launches of a prepared decode: the plan (unless a fused step's prologue made it), the
// attention kernel, and the merge where some row has more than one partition.
// timed: record the optional per-kernel timing events (their creation allocates host-side event
// objects, so the entry point that allocates nothing passes false).
int decode_launch(const DecodeLaunch& L, bool plan, hipStream_t st, bool timed = true) {
  if (L.empty) return PKV_OK;
  const DecodeArgs& a = L.a;
  auto before = [&](int k) { if (timed) timing_before(k, st); };
  auto after = [&](int k) { if (timed) timing_after(k, st); };
  hipError_t e;
  if (plan) {
    before(PKV_K_DECODE_PLAN);
    e = launch_decode_plan(a, L.kv_dtype, L.head_dim, st);
    after(PKV_K_DECODE_PLAN);
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  before(PKV_K_DECODE);
  e = launch_decode_main(a, L.kv_dtype, L.kv_fp8, L.head_dim, L.path, L.pol, L.grid, st);
  after(PKV_K_DECODE);
  if (e != hipSuccess) return PKV_ERR_HIP;
  if (a.max_parts > 1) {
    before(PKV_K_DECODE_REDUCE);
    e = launch_decode_reduce(a, L.kv_dtype, L.head_dim, st);
    after(PKV_K_DECODE_REDUCE);
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

int decode_impl(void* out, int out_dtype, const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                bool kv_fp8, float k_scale, float v_scale, const int32_t* block_tables,
                int32_t block_table_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t n_q_heads,
                int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                int32_t max_seq_len, int32_t partition_size, void* workspace, size_t workspace_bytes,
                uint32_t flags, void* stream, int32_t flat_bps = 0) {
  DecodeLaunch L;
  const int r = decode_prepare(&L, out, out_dtype, q, q_dtype, k_pool, v_pool, kv_fp8, k_scale, v_scale, block_tables,
                               block_table_stride, seq_lens, num_seqs, n_q_heads, n_kv_heads, head_dim, block_size,
                               num_blocks, scale, max_seq_len, partition_size, workspace, workspace_bytes, flags,
                               flat_bps);
  if (r != PKV_OK) return r;
  return decode_launch(L, true, static_cast<hipStream_t>(stream));
}

// ---- the static scratch of pkv_paged_attention_decode_noalloc ---------------------------------
// Device memory for the decode's plan, counters and partial results when the caller cannot
// allocate: a file-scope device array of PKV_STATIC_SCRATCH_BYTES, one copy per GPU, held from the
// code object's load on that GPU until the process ends.  In host code `scratch` names a host-side
// stand-in, never device memory: only the address hipGetSymbolAddress returns for the current
// device may reach a kernel.
static __device__ __align__(256) unsigned char scratch[PKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};   // scratch's device address on each device, once looked up

// The current device's copy of scratch; looked up once per device, with that device current.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attention_decode_noalloc(void* out, int out_dtype, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* block_tables,
                                       int32_t block_table_stride, const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, float scale, int32_t max_seq_len,
                                       int32_t partition_size, int kv_dtype, uint32_t flags, void* stream) {
  // the size check is plain arithmetic and comes first: a call that cannot fit touches no device
  const size_t need = pkv_paged_attention_workspace_size(num_seqs, n_q_heads, head_dim, max_seq_len,
                                                         partition_size);
  if (need > PKV_STATIC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  void* ws = nullptr;
  const int r = scratch_address(&ws);
  if (r != PKV_OK) return r;
  DecodeLaunch L;
  const int c = decode_prepare(&L, out, out_dtype, q, kv_dtype, k_pool, v_pool, false, 1.f, 1.f, block_tables,
                               block_table_stride, seq_lens, num_seqs, n_q_heads, n_kv_heads, head_dim,
                               block_size, num_blocks, scale, max_seq_len, partition_size, ws,
                               PKV_STATIC_SCRATCH_BYTES, flags);
  if (c != PKV_OK) return c;
  // the plan kernel writes every counter and unit the attention reads, and every partial is written
  // before the merge reads it, so nothing in scratch needs clearing between calls
  return decode_launch(L, true, static_cast<hipStream_t>(stream), false);
}

int pkv_paged_attention_decode_ex(void* out, int out_dtype, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables, int32_t block_table_stride,
                                  const int32_t* seq_lens, int32_t num_seqs, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, int32_t max_seq_len, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, int kv_dtype, uint32_t flags,
                                  void* stream) {
  return decode_impl(out, out_dtype, q, kv_dtype, k_pool, v_pool, false, 1.f, 1.f, block_tables,
                     block_table_stride, seq_lens, num_seqs, n_q_heads, n_kv_heads, head_dim, block_size,
                     num_blocks, scale, max_seq_len, partition_size, workspace, workspace_bytes, flags, stream);
}

int pkv_paged_attention_decode_flat(void* out, int out_dtype, const void* q, const void* k_base, const void* v_base,
                                    const int32_t* span_ids, int32_t blocks_per_span, const int32_t* seq_lens,
                                    int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, float scale, int32_t max_seq_len,
                                    int32_t partition_size, void* workspace, size_t workspace_bytes, int kv_dtype,
                                    uint32_t flags, void* stream) {
  if (blocks_per_span <= 0) return PKV_ERR_INVALID;
  return decode_impl(out, out_dtype, q, kv_dtype, k_base, v_base, false, 1.f, 1.f, span_ids, 1, seq_lens,
                     num_seqs, n_q_heads, n_kv_heads, head_dim, block_size, num_blocks, scale, max_seq_len,
                     partition_size, workspace, workspace_bytes, flags, stream, blocks_per_span);
}

int pkv_paged_attention_decode_fp8(void* out, int out_dtype, const void* q, int q_dtype, const void* k_pool,
                                   const void* v_pool, float k_scale, float v_scale, const int32_t* block_tables,
                                   int32_t block_table_stride, const int32_t* seq_lens, int32_t num_seqs,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t num_blocks, float scale, int32_t max_seq_len, int32_t partition_size,
                                   void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  return decode_impl(out, out_dtype, q, q_dtype, k_pool, v_pool, true, k_scale, v_scale, block_tables,
                     block_table_stride, seq_lens, num_seqs, n_q_heads, n_kv_heads, head_dim, block_size,
                     num_blocks, scale, max_seq_len, partition_size, workspace, workspace_bytes, flags, stream);
}

int pkv_paged_attention_decode_v2(const pkv_decode_args* p, void* stream) {
  if (!p || (p->kv_fp8 != 0 && p->kv_fp8 != 1)) return PKV_ERR_INVALID;
  DecodeLaunch L;
  const int r = decode_prepare(&L, p->out, p->out_dtype, p->q, p->q_dtype, p->k_pool, p->v_pool, p->kv_fp8 == 1,
                               p->k_scale, p->v_scale, p->block_tables, p->block_table_stride, p->seq_lens,
                               p->num_seqs, p->n_q_heads, p->n_kv_heads, p->head_dim, p->block_size, p->num_blocks,
                               p->scale, p->max_seq_len, p->partition_size, p->workspace, p->workspace_bytes,
                               p->flags, 0, p->shared_prefix_tokens);
  if (r != PKV_OK) return r;
  return decode_launch(L, true, static_cast<hipStream_t>(stream));
}

int pkv_decode_step(const pkv_decode_step_args* p, void* stream) {
  if (!p) return PKV_ERR_INVALID;
  // ---- the scatter's checks (one new token per row, rows of dtype)
  const int dtype = p->dtype;
  if (!valid_dtype(dtype) || (p->kv_fp8 != 0 && p->kv_fp8 != 1)) return PKV_ERR_INVALID;
  const bool fp8 = p->kv_fp8 == 1;
  if (p->num_seqs < 0 || p->n_kv_heads <= 0 || p->head_dim <= 0) return PKV_ERR_INVALID;
  const int es = esize(dtype);
  if (p->head_dim % (fp8 ? 16 : 16 / es)) return PKV_ERR_INVALID;
  const int64_t row = static_cast<int64_t>(p->n_kv_heads) * p->head_dim;
  const int64_t ks = p->k_token_stride == 0 ? row : p->k_token_stride;
  const int64_t vs = p->v_token_stride == 0 ? row : p->v_token_stride;
  if (ks < row || vs < row || (ks * es) % 16 || (vs * es) % 16) return PKV_ERR_INVALID;
  if (p->num_seqs > 0) {   // the new rows and the slot mapping (an empty step reads neither)
    if (!p->k || !p->v || !aligned(p->k, 16) || !aligned(p->v, 16)) return PKV_ERR_INVALID;
    if (!p->slot_mapping || !aligned(p->slot_mapping, 8) || p->block_table_stride <= 0) return PKV_ERR_INVALID;
  }
  // ---- the decode's checks (the append's are among them: positive block size, a table stride that
  // holds max_seq_len tokens), then its kernel arguments
  DecodeLaunch L;
  const int r = decode_prepare(&L, p->out, p->out_dtype, p->q, dtype, p->k_pool, p->v_pool, fp8, p->k_scale,
                               p->v_scale, p->block_tables, p->block_table_stride, p->seq_lens, p->num_seqs,
                               p->n_q_heads, p->n_kv_heads, p->head_dim, p->block_size, p->num_blocks, p->scale,
                               p->max_seq_len, p->partition_size, p->workspace, p->workspace_bytes, p->flags, 0,
                               p->shared_prefix_tokens);
  if (r != PKV_OK) return r;
  if (L.empty) return PKV_OK;
  const void* slots = nullptr;
  if (!kernel_address(p->slot_mapping, &slots)) return PKV_ERR_INVALID;   // pageable host memory, or no memory
  ScatterArgs sc{p->k, p->v, static_cast<const int64_t*>(slots), p->k_pool, p->v_pool, ks, vs, p->num_seqs,
                 p->num_blocks, p->n_kv_heads, p->head_dim, p->block_size};
  StepArgs sa{static_cast<const int64_t*>(slots), p->block_tables, p->seq_lens, fp8 ? p->k_scale : 1.f,
              fp8 ? p->v_scale : 1.f};
  hipStream_t st = static_cast<hipStream_t>(stream);
  timing_before(PKV_K_STEP_PROLOGUE, st);
  const hipError_t e = launch_step_prologue(L.a, sc, sa, dtype, fp8, p->head_dim, st);
  timing_after(PKV_K_STEP_PROLOGUE, st);
  if (e != hipSuccess) return PKV_ERR_HIP;
  return decode_launch(L, false, st);
}

int pkv_check_block_tables(const int32_t* block_tables, int32_t block_table_stride, const int32_t* seq_lens,
                           int32_t num_seqs, int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                           int32_t* result, void* stream) {
  if (num_seqs < 0 || block_table_stride <= 0 || block_size <= 0 || num_blocks <= 0 || max_seq_len < 0 || !result ||
      !aligned(result, 4))
    return PKV_ERR_INVALID;
  if (num_seqs > 0 && (!block_tables || !seq_lens || !aligned(block_tables, 4) || !aligned(seq_lens, 4)))
    return PKV_ERR_INVALID;
  if ((static_cast<int64_t>(max_seq_len) + block_size - 1) / block_size > block_table_stride) return PKV_ERR_INVALID;
  return launch_check_tables(block_tables, block_table_stride, seq_lens, num_seqs, block_size, num_blocks,
                             max_seq_len, result, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

int pkv_validate_block_tables(const int32_t* block_tables, int32_t block_table_stride, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                              int64_t* bad_entries, int32_t* first_bad_row) {
  if (num_seqs < 0 || block_table_stride <= 0 || block_size <= 0 || num_blocks <= 0 || max_seq_len < 0)
    return PKV_ERR_INVALID;
  if (num_seqs > 0 && (!block_tables || !seq_lens)) return PKV_ERR_INVALID;
  if ((static_cast<int64_t>(max_seq_len) + block_size - 1) / block_size > block_table_stride) return PKV_ERR_INVALID;
  int64_t bad = 0;
  int32_t first = -1;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = seq_lens[s] < 0 ? 0 : (seq_lens[s] > max_seq_len ? max_seq_len : seq_lens[s]);
    const int32_t nb = (L + block_size - 1) / block_size;
    for (int32_t i = 0; i < nb; ++i) {
      const int32_t id = block_tables[static_cast<int64_t>(s) * block_table_stride + i];
      if (id < 0 || id >= num_blocks) {
        ++bad;
        if (first < 0) first = s;
      }
    }
  }
  if (bad_entries) *bad_entries = bad;
  if (first_bad_row) *first_bad_row = first;
  return bad ? PKV_ERR_INVALID : PKV_OK;
}

int pkv_timing_enable(int enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.drop_pending();
  t.enabled = enable != 0;
  return PKV_OK;
}

int pkv_timing_select(uint32_t mask) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.drop_pending();
  t.mask = mask;
  return PKV_OK;
}

int pkv_timing_collect(pkv_kernel_time* out, int32_t cap, int32_t* n) {
  if (cap < 0 || (cap > 0 && !out)) return PKV_ERR_INVALID;
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  double total[PKV_K_COUNT] = {0};
  int32_t count[PKV_K_COUNT] = {0};
  int status = PKV_OK;
  for (auto& r : t.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      status = PKV_ERR_HIP;
      continue;
    }
    total[r.kernel] += ms;
    count[r.kernel] += 1;
  }
  t.drop_pending();
  int32_t m = 0;
  for (int k = 0; k < PKV_K_COUNT; ++k) {
    if (!count[k]) continue;
    if (m < cap) out[m] = pkv_kernel_time{k, count[k], total[k]};
    ++m;
  }
  if (n) *n = m;
  return status;
}

}  // extern "C"
