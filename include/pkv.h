/*
 * libpagedkv -- paged KV cache for decode on AMD Instinct MI355X (gfx950).
 *
 * The KV cache of every sequence lives in fixed-size physical blocks of B
 * tokens taken from one device pool; a per-sequence block table maps
 * logical block i (tokens i*B .. (i+1)*B-1) to the physical block that backs
 * it, and blocks are handed out only when a sequence fills its last one
 * ("PagedAttention -- Math + Memory Model", section "PagedAttention: blocks
 * and the block table").  Decode attention follows that table and gathers
 * the scattered blocks for QK^T, a numerically stable softmax and the
 * value-weighted sum (same section; "KV-cache paging in vLLM", section "The
 * Attention Kernel Change").
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Return value: PKV_OK or a negative PKV_ERR_* code.  Argument checks run
 *   before anything is launched or changed; a rejected call has no effect.
 * - Device pointers are caller-owned.  The library never allocates device
 *   memory: scratch space is the caller's workspace argument, except for
 *   pkv_paged_attention_decode_noalloc, whose scratch is a static device array
 *   of the library (PKV_STATIC_SCRATCH_BYTES per GPU).
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Launches are asynchronous on that stream; nothing here synchronises.
 *   A failed launch returns PKV_ERR_HIP.
 * - Element types: PKV_F32 (float), PKV_F16 (IEEE binary16), PKV_BF16
 *   (bfloat16).  Copies move raw bits (NaN payloads and -0.0 survive).
 *   A quantised cache holds PKV_FP8_E4M3 codes in its pools (see the FP8
 *   section below); rows, q and results are never FP8.
 * - Integer sizes are int32_t, token slots are int64_t.
 *
 * Storage layout of the pools (row-major, X = 16 bytes / element size, so X
 * elements make one 16-byte vector):
 *   key pool   [num_blocks][n_kv_heads][head_dim / X][block_size][X]
 *   value pool [num_blocks][n_kv_heads][head_dim][block_size]
 * One physical block holds all KV heads of its B tokens; the (block, head)
 * chunk of each pool is block_size * head_dim elements, contiguous.  Slot s
 * is token s % block_size of block s / block_size.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes and element types --------------------------------------- */
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,     /* a null pointer, size out of range, inconsistent shapes */
  PKV_ERR_OOM = -2,         /* the allocator's pool has too few free blocks */
  PKV_ERR_NOT_FOUND = -3,   /* unknown sequence id */
  PKV_ERR_UNSUPPORTED = -4, /* valid, but no kernel for this head_dim / block_size / group */
  PKV_ERR_HIP = -5,         /* the HIP runtime reported an error */
  PKV_ERR_SCRATCH = -6      /* pkv_paged_attention_decode_noalloc: the call needs more scratch than
                               PKV_STATIC_SCRATCH_BYTES */
};

enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3 };

/* Kernel ids reported by pkv_timing_collect. */
enum {
  PKV_K_RESHAPE_AND_CACHE = 0,
  PKV_K_APPEND_SLOTS = 1,
  PKV_K_DECODE_PLAN = 2,
  PKV_K_DECODE = 3,
  PKV_K_DECODE_REDUCE = 4,
  PKV_K_COPY_BLOCKS = 5,
  PKV_K_SWAP_BLOCKS = 6,
  PKV_K_STEP_PROLOGUE = 7,
  PKV_K_COUNT = 8
};

/* Text for a status code (static storage, never NULL). */
const char* pkv_status_string(int status);

/* Library ABI version, bumped on any incompatible change (2: pkv_decode_step_args gained
 * shared_prefix_tokens). */
int pkv_version(void);

/* Bytes of ONE pool (key or value) for the given shape and pool element type (PKV_FP8_E4M3
 * included); 0 if the shape is invalid. */
size_t pkv_pool_bytes(int32_t num_blocks, int32_t n_kv_heads, int32_t head_dim,
                      int32_t block_size, int dtype);

/* ---- slot-mapping scatter ---------------------------------------------------
 * Writes each new token's key and value rows into its physical slot:
 *   for every token t with 0 <= slot_mapping[t] < num_blocks * block_size,
 *     key pool   element (slot/B, h, d/X, slot%B, d%X) = k[t, h, d]
 *     value pool element (slot/B, h, d,   slot%B)      = v[t, h, d]
 * Negative slots (padding tokens) and slots past the pool are skipped.  The
 * append of a token to its sequence's last block is what the block manager
 * hands out slots for ("PagedAttention -- Math + Memory Model", section
 * "PagedAttention: blocks and the block table"; "KV-Cache Optimization &
 * PagedAttention for Long-Context Agents", section "Key KV-Cache Optimization
 * Principles", item 1).
 *   k, v          device, [num_tokens][n_kv_heads][head_dim] with a token stride
 *                 of k_token_stride / v_token_stride elements (0 = n_kv_heads*head_dim;
 *                 lets k and v be views into a fused QKV buffer; 16-byte aligned rows)
 *   slot_mapping  device, int64 [num_tokens]
 *   k_pool/v_pool device, pools of the documented layout
 * Two tokens with the same slot in one call: undefined which one lands.
 * Bits are copied unchanged.  head_dim must be a multiple of X.  dtype: PKV_F32,
 * PKV_F16 or PKV_BF16 (FP8 pools take pkv_reshape_and_cache_fp8). */
int pkv_reshape_and_cache(const void* k, const void* v, const int64_t* slot_mapping,
                          int32_t num_tokens, int64_t k_token_stride, int64_t v_token_stride,
                          void* k_pool, void* v_pool, int32_t num_blocks, int32_t n_kv_heads,
                          int32_t head_dim, int32_t block_size, int dtype, void* stream);

/* ---- copy-on-write block copies ----------------------------------------------------
 * For every pair i, block pairs[2i+1] (dst) of both pools becomes a bit copy of block
 * pairs[2i] (src), every KV head ("PagedAttention -- Math + Memory Model", section
 * "Copy-on-write: sharing blocks across samples": a sequence about to write into a block
 * it shares with another gets a private copy, and its write goes to the copy).  The pairs
 * are the ones pkv_alloc / pkv_alloc_batch return; apply them before the scatter of the
 * tokens whose append produced them.  A pair with an id outside [0, num_blocks), or with
 * src == dst, is skipped (no fault).  Destinations must be distinct and never a source in
 * the same call (the allocator's pairs always are: a destination is a fresh block), since
 * the pairs are copied concurrently.
 *   pairs          device int32 [n_pairs][2], (src, dst)
 *   k_pool, v_pool device pools of the documented layout, 16-byte aligned, updated in place
 * One block of one pool is n_kv_heads * head_dim * block_size elements of dtype (any pool
 * type, PKV_FP8_E4M3 included); that byte count must be a multiple of 16
 * (PKV_ERR_UNSUPPORTED otherwise). */
int pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n_pairs,
                    int32_t num_blocks, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                    int dtype, void* stream);

/* ---- block moves between a pool and host swap space ---------------------------------
 * For every pair i, block pairs[2i+1] of the destination arrays (dst_k, dst_v) becomes a bit copy
 * of block pairs[2i] of the source arrays (src_k, src_v), both pools.  The arrays hold blocks of
 * the documented pool layout (one block = n_kv_heads * head_dim * block_size elements); each is
 * device memory or pinned host memory from hipHostMalloc (a torch tensor with pin_memory), which
 * the kernel reads or writes over the host link.  The pairs come from pkv_swap_out (pool -> host)
 * or pkv_swap_in (host -> pool).  Pairs with an id outside [0, src_blocks) / [0, dst_blocks) are
 * skipped; destinations must be distinct.  Any pointer that is neither device nor pinned host
 * memory is PKV_ERR_INVALID, checked before the launch.  pairs: int32 [n_pairs][2], device or
 * pinned host memory. */
int pkv_swap_blocks(const void* src_k, const void* src_v, int32_t src_blocks, void* dst_k, void* dst_v,
                    int32_t dst_blocks, const int32_t* pairs, int32_t n_pairs, int32_t n_kv_heads,
                    int32_t head_dim, int32_t block_size, int dtype, void* stream);

/* ---- device half of the on-demand append --------------------------------------
 * One decode step appends one token per batch row.  For every row i with
 * slot_mapping[i] >= 0, with p = seq_lens[i] (the new token's position):
 *   block_tables[i * block_table_stride + p / block_size] = slot_mapping[i] / block_size
 *   seq_lens[i] = p + 1
 * i.e. the physical block the host allocator chose for position p is
 * appended to (or kept in) the row's table ("PagedAttention -- Math + Memory
 * Model", section "PagedAttention: blocks and the block table": a sequence
 * that fills its last block gets one more from the pool, appended to its
 * table).  Rows with a negative slot, a negative length or p / block_size >=
 * block_table_stride are left unchanged.
 *   slot_mapping  device int64 [num_seqs]
 *   block_tables  device int32 [num_seqs][block_table_stride], updated in place
 *   seq_lens      device int32 [num_seqs], updated in place */
int pkv_append_slots(const int64_t* slot_mapping, int32_t num_seqs, int32_t* block_tables,
                     int32_t block_table_stride, int32_t* seq_lens, int32_t block_size,
                     void* stream);

/* ---- decode attention ---------------------------------------------------------
 * For every batch row s and query head h (G = n_q_heads / n_kv_heads, KV head
 * kv = h / G, L = seq_lens[s]):
 *   x_j  = scale * <q[s,h,:], K_s[j,kv,:]>               j = 0 .. L-1
 *   out[s,h,:] = sum_j exp(x_j - max x) V_s[j,kv,:] / sum_j exp(x_j - max x)
 * where K_s[j] / V_s[j] is token j % B of physical block
 * block_tables[s * block_table_stride + j / B].  Rows with L <= 0 get zeros.
 *
 * Work is split into partitions of partition_size tokens per (row, KV head);
 * each partition keeps its running max, sum and fp32 accumulator, and rows
 * with more than one partition are merged by log-sum-exp rescaling.
 * Accumulation is fp32; for 16-bit KV the products run on MFMA
 * with the softmax weights rounded to the KV type (the denominator sums the
 * same rounded weights).
 *   out            device [num_seqs][n_q_heads][head_dim] of out_dtype
 *                  (out_dtype = kv_dtype or PKV_F32; rounding to nearest even)
 *   q              device [num_seqs][n_q_heads][head_dim] of kv_dtype, 16-byte aligned rows
 *   k_pool, v_pool device pools of the documented layout
 *   block_tables   device int32 [num_seqs][block_table_stride]; only the first
 *                  ceil(L/B) entries of a row are read; an entry outside
 *                  [0, num_blocks) is clamped into it (no fault; the row's result is
 *                  then meaningless: pkv_check_block_tables / pkv_validate_block_tables
 *                  report such entries)
 *   seq_lens       device int32 [num_seqs]; a length above max_seq_len is treated as
 *                  max_seq_len
 *   max_seq_len    host bound on seq_lens, sizes the workspace
 *   partition_size tokens per partition: a positive multiple of 32, or 0 for
 *                  "never split" (one partition of max_seq_len tokens)
 *   workspace      device scratch of at least pkv_paged_attention_workspace_size()
 *                  bytes, 256-byte aligned; its contents on entry do not matter; two
 *                  calls in flight at once must not share it
 * Supported: head_dim 64 or 128; block_size 8, 16 or 32; G = 1..16 for
 * 16-bit KV (MFMA, heads padded to 16), G = 1..4 for fp32 KV.  kv_dtype is the
 * type of q and of the pools (PKV_F32, PKV_F16 or PKV_BF16; FP8 pools take
 * pkv_paged_attention_decode_fp8). */
size_t pkv_paged_attention_workspace_size(int32_t num_seqs, int32_t n_q_heads, int32_t head_dim,
                                          int32_t max_seq_len, int32_t partition_size);

int pkv_paged_attention_decode(void* out, int out_dtype, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_tables,
                               int32_t block_table_stride, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               float scale, int32_t max_seq_len, int32_t partition_size,
                               void* workspace, size_t workspace_bytes, int kv_dtype,
                               void* stream);

/* pkv_paged_attention_decode with flags (pkv_paged_attention_decode is this with flags = 0).
 *   PKV_DECODE_SHARED_KV  some blocks are read by more than one row of the batch (forked
 *                         samples, a shared prompt): keep key/value lines cacheable so the
 *                         rows that reread them hit in L2 / the Infinity Cache.  Without it
 *                         the tiles are streamed with the non-temporal hint, which is faster
 *                         when every block is read once.  It changes no result.
 *   PKV_DECODE_VECTOR     16-bit KV with G = 1 (multi-head attention): per-token fp32 dot products
 *                         with cross-lane reductions and fp32 weights, instead of MFMA with the one
 *                         head padded to 16 (within the same tolerance of the exact result, not the
 *                         same bits); PKV_ERR_UNSUPPORTED for G > 1, FP8 pools and flat spans.
 * Unknown flag bits: PKV_ERR_INVALID. */
enum { PKV_DECODE_SHARED_KV = 1, PKV_DECODE_VECTOR = 2 };
int pkv_paged_attention_decode_ex(void* out, int out_dtype, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables, int32_t block_table_stride,
                                  const int32_t* seq_lens, int32_t num_seqs, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, int32_t max_seq_len, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, int kv_dtype, uint32_t flags,
                                  void* stream);

/* ---- finding a bad block table -------------------------------------------------------------------
 * Decode reads, for row s, the block ids block_tables[s * stride + i], i < ceil(L / B), and an id
 * outside [0, num_blocks) is clamped into the pool so that no access faults: the row's result is then
 * meaningless and nothing reports it ("PagedAttention -- Math + Memory Model", section "PagedAttention:
 * blocks and the block table": each of a sequence's logical blocks maps to a physical block of the
 * pool).  These two calls report such entries instead; L is seq_lens[s] clamped to [0, max_seq_len] as
 * decode clamps it, and block_table_stride must hold ceil(max_seq_len / B) entries.
 *
 * pkv_validate_block_tables: host arrays, checked on the CPU.  PKV_OK if every read entry is in the
 * pool, else PKV_ERR_INVALID with *bad_entries = the number of out-of-pool entries and *first_bad_row =
 * the first row holding one (-1 if none; both outputs nullable).
 *
 * pkv_check_block_tables: device arrays, checked by a kernel on `stream` (no allocation, no memset, so
 * it may be captured in a graph).  It writes result[0] = the number of out-of-pool entries and
 * result[1] = the first row holding one (INT32_MAX if none) to the caller's device int32 [2]; the
 * caller reads them after the stream reaches that point.  Nothing traps on the GPU. */
int pkv_validate_block_tables(const int32_t* block_tables, int32_t block_table_stride, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                              int64_t* bad_entries, int32_t* first_bad_row);
int pkv_check_block_tables(const int32_t* block_tables, int32_t block_table_stride, const int32_t* seq_lens,
                           int32_t num_seqs, int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                           int32_t* result, void* stream);

/* ---- decode attention without allocation --------------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  pkv_paged_attention_decode_ex with the same arguments, except that
 * the plan, the counters and the partial results live in the library's own static scratch, a device
 * array of PKV_STATIC_SCRATCH_BYTES on each GPU, instead of a workspace argument.  The call allocates
 * nothing (no hipMalloc, no library allocation, no timing events); its first call on a device looks up
 * that device's copy of the scratch (hipGetSymbolAddress), which the device then holds until the process
 * ends.  Same kernels and the same bits as pkv_paged_attention_decode_ex.
 *   - A call whose pkv_paged_attention_workspace_size() exceeds PKV_STATIC_SCRATCH_BYTES returns
 *     PKV_ERR_SCRATCH before touching the device (128 MiB holds, e.g., 256 rows x 64 query heads x
 *     128 dims up to 32768 tokens in 3072-token partitions, or 8 rows of 65536 tokens in 512-token
 *     partitions).
 *   - Every call on one GPU shares that GPU's scratch, and each call rewrites what it reads (no
 *     clearing is needed between calls).  Two calls in flight at once on one GPU (other streams,
 *     other threads) race on it: callers must order them.
 * FP8 pools are not taken here (use pkv_paged_attention_decode_fp8 with a workspace). */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
int pkv_paged_attention_decode_noalloc(void* out, int out_dtype, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* block_tables,
                                       int32_t block_table_stride, const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, float scale, int32_t max_seq_len,
                                       int32_t partition_size, int kv_dtype, uint32_t flags, void* stream);

/* ---- measurement: the streaming-read ceiling ---------------------------------------------------
 * Reads a device buffer once with waves shaped like the decode kernel's (one 64-lane wave per
 * workgroup, 16 bytes per lane per load) and computes nothing on the data, so that the decode
 * kernel's bandwidth can be set beside what HBM delivers to such waves on this GPU, next to the data
 * sheet's figure.  Not part of the decode path.
 *   buf, bytes      device buffer (16-byte aligned) and its size; at most `bytes` are read
 *   waves_per_cu    1..32 single-wave workgroups per compute unit
 *   loads_per_batch 4, 8 or 16 loads of 1 KiB per wave per batch; two batches in flight per wave
 *   mode            bit 0: non-temporal loads; bit 1: 4 KiB chunks in a scattered order (as paged
 *                   blocks are), else each wave reads one contiguous span
 *   sink            device uint32 [1024], written only in a case that never arises (keeps the loads)
 *   bytes_read      host, receives the bytes the launch reads (for the bandwidth)
 * Asynchronous on `stream`; PKV_ERR_INVALID for a buffer too small for one batch of every wave. */
int pkv_read_probe(const void* buf, size_t bytes, int32_t waves_per_cu, int32_t loads_per_batch, int mode,
                   uint32_t* sink, size_t* bytes_read, void* stream);

/* ---- decode attention: every option in one call ------------------------------------------------
 * The decode of pkv_paged_attention_decode_ex (16-bit or fp32 pools) or pkv_paged_attention_decode_fp8
 * (kv_fp8 = 1: FP8 E4M3 pools under k_scale / v_scale, q of q_dtype), with one more choice of how the
 * pools are read:
 *   shared_prefix_tokens  0, or n > 0: the first n tokens of every row lie in blocks that other rows of
 *                         the batch read too (a prompt the rows were forked from, "KV-cache paging in
 *                         vLLM", section "What This Changes in Practice": the shared blocks are
 *                         physically shared, not copied).  Tiles of 16-bit and FP8 pools that start
 *                         before token n are read with cacheable loads, so the rows that re-read them
 *                         hit L2 and the Infinity Cache, and every later tile is streamed with the
 *                         non-temporal hint, so a row's private tokens neither evict the shared ones nor
 *                         pay for the write-back of dirty lines they would evict.  The choice is made per
 *                         tile, with no change to any result.  It overrides PKV_DECODE_SHARED_KV (which
 *                         reads every tile cacheable); on the vector path it reads every tile cacheable;
 *                         flat spans: PKV_ERR_UNSUPPORTED.
 * Every other field means what the argument of that name means for the calls above. */
typedef struct {
  void* out;
  int32_t out_dtype;
  const void* q;
  int32_t q_dtype;
  const void* k_pool;
  const void* v_pool;
  int32_t kv_fp8;
  float k_scale;
  float v_scale;
  const int32_t* block_tables;
  int32_t block_table_stride;
  const int32_t* seq_lens;
  int32_t num_seqs;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  float scale;
  int32_t max_seq_len;
  int32_t partition_size;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
  int32_t shared_prefix_tokens;
} pkv_decode_args;

int pkv_paged_attention_decode_v2(const pkv_decode_args* args, void* stream);

/* ---- quantised cache: FP8 E4M3 pools ------------------------------------------------
 * Quantising the cached keys and values is the memory lever the pages put after paging: an
 * 8-bit cache halves the bytes each sequence's attention reads ("Contiguous vs Paged KV Cache
 * on RDNA4", section "The order of the memory levers"; "KV-Cache Optimization & PagedAttention
 * for Long-Context Agents", introduction).  The format is OCP FP8 E4M3: sign, 4 exponent bits
 * (bias 7), 3 mantissa bits, no infinities, S.1111.111 = NaN, largest finite 448.  Each pool
 * has one per-tensor scale: an element x is stored as code(x / scale) and represents
 * scale * value(code).  The pools keep the documented layout with one-byte elements, so
 * X = 16 codes per key vector and head_dim must be a multiple of 16. */

/* The scatter of pkv_reshape_and_cache into FP8 pools: for every token t with an in-range
 * slot, each element x of k[t] / v[t] (src_dtype: PKV_F32, PKV_F16 or PKV_BF16) is stored as
 * the E4M3 code of x / k_scale (x / v_scale for values): the quotient is the fp32 IEEE
 * division of the fp32 value of x, then the nearest code, ties to the even mantissa;
 * magnitudes of 448 and above become +-448 and NaN becomes 0x7F.  Strides, alignment and
 * skipped slots as for pkv_reshape_and_cache (strides in src_dtype elements).  Scales must be
 * positive and finite (PKV_ERR_INVALID otherwise). */
int pkv_reshape_and_cache_fp8(const void* k, const void* v, const int64_t* slot_mapping,
                              int32_t num_tokens, int64_t k_token_stride, int64_t v_token_stride,
                              void* k_pool, void* v_pool, int32_t num_blocks, int32_t n_kv_heads,
                              int32_t head_dim, int32_t block_size, int src_dtype, float k_scale,
                              float v_scale, void* stream);

/* Decode attention over FP8 pools: pkv_paged_attention_decode_ex on the values the pools
 * represent, K = k_scale * value(code), V = v_scale * value(code).
 *   q        device [num_seqs][n_q_heads][head_dim] of q_dtype (PKV_BF16 or PKV_F16; PKV_F32:
 *            PKV_ERR_UNSUPPORTED), 16-byte aligned rows
 *   out      of out_dtype = q_dtype or PKV_F32
 * The codes are widened exactly to q_dtype in registers and the products run on MFMA with fp32
 * accumulation; k_scale is folded into the score scale (scale * k_scale, rounded to fp32) and
 * v_scale multiplies the accumulated values.  The softmax weights are rounded to q_dtype for the
 * value product, as for 16-bit pools.  Scales must be positive and finite.  Supported shapes,
 * flags, workspace and every other argument as for pkv_paged_attention_decode_ex (G = 1..16). */
int pkv_paged_attention_decode_fp8(void* out, int out_dtype, const void* q, int q_dtype,
                                   const void* k_pool, const void* v_pool, float k_scale, float v_scale,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t num_blocks, float scale, int32_t max_seq_len,
                                   int32_t partition_size, void* workspace, size_t workspace_bytes,
                                   uint32_t flags, void* stream);

/* ---- a whole decode step in fewer launches -----------------------------------------------------
 * One decode step of a batch: every row appends one token and attends over all of its tokens
 * ("PagedAttention -- Math + Memory Model", section "PagedAttention: blocks and the block table":
 * the new token's key and value go to its slot, its block is recorded in the row's table, and the
 * attention then reads every token through the table).  The result is exactly that of
 *   pkv_append_slots(slot_mapping, ...);
 *   pkv_reshape_and_cache(k, v, slot_mapping, num_tokens = num_seqs, ...)   (kv_fp8: _fp8);
 *   pkv_paged_attention_decode_ex(...)                                       (kv_fp8: _fp8);
 * on one stream: the same bits in the pools, the block tables, the lengths and the output.  It runs
 * as one prologue kernel (one workgroup appends and then plans the attention's work over the new
 * lengths while the others scatter), the attention kernel and, when a row spans more than one
 * partition, the merge: three fewer launches than the separate calls.
 *   slot_mapping   int64 [num_seqs]: the slot of row s's new token (token s of k and v), as the
 *                  allocator gave it; a negative slot skips the row's scatter and append.  Device
 *                  memory or pinned host memory (hipHostMalloc): the prologue reads
 *                  host memory over the host link (each slot once for the append and once per
 *                  scatter workgroup that covers its token), so the step needs no copy.
 *                  It must not change until the prologue has run.  Pageable host memory:
 *                  PKV_ERR_INVALID.
 *   k, v           device rows, token s of each at s * k_token_stride (v_token_stride) elements of
 *                  dtype, n_kv_heads * head_dim elements each; strides 0 = packed; 16-byte aligned
 *   kv_fp8         0: the pools hold dtype; 1: they hold FP8 E4M3 codes under k_scale / v_scale
 *                  (dtype PKV_F16 or PKV_BF16)
 *   block_tables, seq_lens  device, updated by the append and then read by the attention
 *   dtype          the type of k, v and q (and of out unless out_dtype is PKV_F32)
 * Every other field as for pkv_paged_attention_decode_ex / pkv_paged_attention_decode_fp8.  The
 * checks are those of the three calls; a rejected step changes nothing. */
typedef struct {
  const void* k;
  const void* v;
  int64_t k_token_stride;
  int64_t v_token_stride;
  const int64_t* slot_mapping;
  void* k_pool;
  void* v_pool;
  int32_t num_blocks;
  int32_t kv_fp8;
  float k_scale;
  float v_scale;
  int32_t* block_tables;
  int32_t* seq_lens;
  int32_t block_table_stride;
  int32_t num_seqs;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  void* out;
  int32_t out_dtype;
  int32_t dtype;
  const void* q;
  float scale;
  int32_t max_seq_len;
  int32_t partition_size;
  uint32_t flags;
  void* workspace;
  size_t workspace_bytes;
  int32_t shared_prefix_tokens;   /* as in pkv_decode_args (0: none) */
} pkv_decode_step_args;

int pkv_decode_step(const pkv_decode_step_args* args, void* stream);

/* ---- flat spans: contiguous virtual ranges backed on demand ------------------------------
 * The alternative to a block table that "Contiguous vs Paged KV Cache on RDNA4" names (sections
 * "Is paging the only way to fix KV cache fragmentation?" and "Why the single-user verdict
 * flipped"): every sequence gets one contiguous virtual range reserved up front, physical memory
 * is mapped into it as the sequence grows, and attention reads the range as a flat span with no
 * block table.
 *
 * A span pool reserves one virtual range per pool (keys, values) and cuts it into max_spans
 * spans.  A span keeps the documented block layout: span s holds blocks s * blocks_per_span ..
 * (s + 1) * blocks_per_span - 1 of a virtual pool of num_blocks = max_spans * blocks_per_span
 * blocks, so token p of span s has slot (s * blocks_per_span + p / B) * B + p % B and
 * pkv_reshape_and_cache / pkv_copy_blocks work on it unchanged (k_base / v_base as the pools).
 * Physical memory comes in chunks of chunk_bytes (0 = 2 MiB; a multiple of the device's allocation
 * granularity), mapped with the HIP virtual memory API.  Only mapped memory may be touched: every
 * slot written and every token a decode reads must lie in a reserved prefix of its span (reading
 * or writing an unmapped part of a span is a GPU memory fault).  A released span's chunks are kept
 * for reuse until pkv_span_pool_trim.  The pool belongs to the device current at creation; it is
 * not thread-safe across threads that also launch on its memory without synchronising. */
typedef struct pkv_span_pool pkv_span_pool;

typedef struct {
  void* k_base;             /* device: the key pool's virtual range */
  void* v_base;             /* device: the value pool's virtual range */
  int32_t blocks_per_span;
  int32_t num_blocks;       /* max_spans * blocks_per_span */
  size_t chunk_bytes;
  size_t span_bytes;        /* one span of one pool: blocks_per_span * block bytes */
  size_t mapped_bytes;      /* physical memory mapped now, both pools */
  size_t spare_bytes;       /* unmapped chunks kept for reuse */
} pkv_span_info;

/* max_tokens: the longest sequence a span must hold (blocks_per_span >= ceil(max_tokens / B); it
 * is rounded up so that a span is a whole number of chunks).  dtype: any pool type.
 * PKV_ERR_UNSUPPORTED if the device has no virtual memory management; PKV_ERR_OOM if the virtual
 * ranges cannot be reserved. */
int pkv_span_pool_create(int32_t max_spans, int32_t max_tokens, int32_t n_kv_heads, int32_t head_dim,
                         int32_t block_size, int dtype, size_t chunk_bytes, pkv_span_pool** out);
void pkv_span_pool_destroy(pkv_span_pool* p);

/* Backs tokens [0, n_tokens) of span (in both pools) with physical memory: maps the missing chunks.
 * All or nothing: PKV_ERR_OOM (no device memory) or PKV_ERR_HIP leaves the span as it was.
 * n_tokens above the span's capacity: PKV_ERR_INVALID.  Never shrinks a span. */
int pkv_span_reserve(pkv_span_pool* p, int32_t span, int32_t n_tokens);

/* Unmaps all of a span's memory (its contents are lost); the chunks are kept for reuse.  Work on the
 * device that still reads or writes the span must have finished. */
int pkv_span_release(pkv_span_pool* p, int32_t span);

/* Frees the chunks kept for reuse. */
int pkv_span_pool_trim(pkv_span_pool* p);

int pkv_span_pool_info(pkv_span_pool* p, pkv_span_info* out);

/* Tokens of span that are backed now (a multiple of B), or -1 for a bad argument. */
int32_t pkv_span_mapped_tokens(pkv_span_pool* p, int32_t span);

/* Decode attention over flat spans: pkv_paged_attention_decode_ex where row s's token j is token
 * j % B of block span_ids[s] * blocks_per_span + j / B, computed in the kernel (no block table is
 * read).  k_base / v_base, num_blocks and blocks_per_span come from pkv_span_pool_info;
 * span_ids is device int32 [num_seqs].  Every row's first seq_lens[s] tokens must be reserved.
 * max_seq_len must fit a span (ceil(max_seq_len / B) <= blocks_per_span).  16-bit KV only
 * (PKV_ERR_UNSUPPORTED for fp32), and PKV_DECODE_SHARED_KV is unsupported (spans are never
 * shared).  The result is bit-identical to pkv_paged_attention_decode_ex over the same tokens. */
int pkv_paged_attention_decode_flat(void* out, int out_dtype, const void* q, const void* k_base,
                                    const void* v_base, const int32_t* span_ids, int32_t blocks_per_span,
                                    const int32_t* seq_lens, int32_t num_seqs, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, float scale, int32_t max_seq_len,
                                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                                    int kv_dtype, uint32_t flags, void* stream);

/* ---- host block allocator ------------------------------------------------------
 * The block manager of the pages: a free list of physical block ids, a
 * reference count per block, and per-sequence block tables.
 *   - free list: blocks are taken from the head and returned to the tail, as
 *     in the simulator of "KV-Cache Optimization & PagedAttention for
 *     Long-Context Agents" (section "Python Implementation: Paged KV-Cache
 *     Virtual Memory Simulator"); a freed sequence returns its blocks in
 *     logical order;
 *   - on-demand append: a new sequence owns zero blocks; position p takes a
 *     fresh block when p % B == 0 ("PagedAttention -- Math + Memory Model",
 *     section "PagedAttention: blocks and the block table");
 *   - sharing and copy-on-write: pkv_fork points a child's first table entries
 *     at the parent's blocks (reference count + 1 each); the first append into a
 *     partly filled block that others still share takes a fresh block, reports
 *     the (old, new) pair for the caller to copy, and drops the old block's count;
 *     a block rejoins the pool when its count reaches zero (same page, section
 *     "Copy-on-write: sharing blocks across samples").
 * Host memory only; an allocator is not thread-safe (one caller at a time).
 * Sequence ids are arbitrary int64 values chosen by the caller. */
typedef struct pkv_allocator pkv_allocator;

typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t free_blocks;
  int32_t allocated_blocks; /* reference count > 0 */
  int32_t shared_blocks;    /* reference count > 1 */
  int32_t reserved;
  int64_t num_seqs;
  int64_t live_tokens;      /* sum of sequence lengths (a shared token counts per sequence) */
  int64_t allocated_slots;  /* allocated_blocks * block_size */
} pkv_stats;

/* initial_free_order: NULL for 0..num_blocks-1, else a permutation of it (the
 * order blocks are handed out in).  *out receives the new allocator. */
int pkv_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                         pkv_allocator** out);
void pkv_allocator_destroy(pkv_allocator* a);

/* Appends n_new_tokens to seq_id (created with zero blocks if unknown).
 * slots_out (nullable, n_new_tokens entries) receives each token's slot.
 * cow_pair_out (nullable, 2 entries) receives [old, new] if the append copied a
 * shared block; *n_cow (nullable) receives 0 or 1.  All or nothing: PKV_ERR_OOM
 * leaves the allocator unchanged (and does not create seq_id). */
int pkv_alloc(pkv_allocator* a, int64_t seq_id, int32_t n_new_tokens, int64_t* slots_out,
              int32_t* cow_pair_out, int32_t* n_cow);

/* pkv_alloc of n_new_each tokens for each of n_seqs distinct sequences, in order,
 * as one all-or-nothing step.  slots_out (nullable) is [n_seqs][n_new_each];
 * cow_pairs_out (nullable) has room for 2 * n_seqs ints and receives the copy
 * pairs in order; *n_cow (nullable) their count.  Repeated ids: PKV_ERR_INVALID. */
int pkv_alloc_batch(pkv_allocator* a, const int64_t* seq_ids, int32_t n_seqs, int32_t n_new_each,
                    int64_t* slots_out, int32_t* cow_pairs_out, int32_t* n_cow);

/* The child (which must not exist) shares the parent's first ceil(n/B) blocks and
 * gets length n; n_shared_tokens = -1 shares the parent's whole length. */
int pkv_fork(pkv_allocator* a, int64_t parent, int64_t child, int32_t n_shared_tokens);

/* Drops seq_id; each of its blocks loses one reference, in logical order, and
 * rejoins the tail of the free list at zero. */
int pkv_free(pkv_allocator* a, int64_t seq_id);

/* Copies up to cap table entries of seq_id to out (nullable); *n_blocks and
 * *seq_len (nullable) receive the full table length and the sequence length. */
int pkv_get_block_table(const pkv_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                        int32_t* n_blocks, int32_t* seq_len);

/* Packs the tables of a batch into tables[n_seqs][stride] (unused entries =
 * pad_value) and their lengths into seq_lens (nullable).  PKV_ERR_INVALID if a
 * table is longer than stride. */
int pkv_fill_block_tables(const pkv_allocator* a, const int64_t* seq_ids, int32_t n_seqs,
                          int32_t* tables, int32_t stride, int32_t pad_value, int32_t* seq_lens);

int pkv_allocator_stats(const pkv_allocator* a, pkv_stats* out);

/* ---- swapping sequences to host memory ---------------------------------------------
 * Instead of evicting a sequence and recomputing its cache, its blocks can move to host memory
 * and come back later ("Reserve for the worst case, or page", section "What this model leaves
 * out").  The allocator manages host_blocks host slots of one block each, with their own FIFO
 * free list (slots 0 .. host_blocks-1 initially, head first).
 *   swap-out: every block of a device-resident sequence, in logical order, takes the next host
 *     slot and gives the pair (device block, host slot); then the sequence's references are
 *     dropped exactly as pkv_free drops them (a block still shared stays on the device for its
 *     other sequences).  The sequence is then swapped out: it keeps its id and length, cannot
 *     append or be forked, and has no block table until it is swapped back in.
 *   swap-in: fresh device blocks are taken in logical order, giving (host slot, device block);
 *     the host slots return, in order, to the tail of their list.  The blocks are private.
 * Both are all or nothing: PKV_ERR_OOM (too few host slots / device blocks) changes nothing.
 * pairs_out needs room for 2 * (the sequence's block count) ints; *n_pairs receives that count
 * on every return, and a smaller cap is PKV_ERR_INVALID (nothing changes).  Apply the pairs with
 * pkv_swap_blocks before the freed blocks (or host slots) are written again: launched on the
 * stream of the later writes, stream order guarantees it.  pkv_free of a swapped-out sequence
 * returns its host slots. */
int pkv_allocator_set_swap_space(pkv_allocator* a, int32_t host_blocks);   /* once per allocator */
int pkv_swap_out(pkv_allocator* a, int64_t seq_id, int32_t* pairs_out, int32_t cap, int32_t* n_pairs);
int pkv_swap_in(pkv_allocator* a, int64_t seq_id, int32_t* pairs_out, int32_t cap, int32_t* n_pairs);
int pkv_swap_stats(const pkv_allocator* a, int32_t* host_blocks, int32_t* host_free, int64_t* swapped_seqs);

/* Reference count of a block, or -1 for an id outside the pool. */
int32_t pkv_block_ref_count(const pkv_allocator* a, int32_t block);

/* The free list from head to tail: up to cap ids into out (nullable), *n = its length. */
int pkv_free_list(const pkv_allocator* a, int32_t* out, int32_t cap, int32_t* n);

/* ---- kernel timing ----------------------------------------------------------------
 * While enabled, every kernel launch of this library is bracketed by a pair of
 * hipEvents recorded on its stream.  pkv_timing_collect waits for those events,
 * writes one record per kernel id that ran (launch count and summed duration)
 * and forgets them.  Enabling or disabling also forgets pending records. */
typedef struct {
  int32_t kernel;
  int32_t launches;
  double total_ms;
} pkv_kernel_time;

int pkv_timing_enable(int enable);
int pkv_timing_collect(pkv_kernel_time* out, int32_t cap, int32_t* n);
/* Restricts timing to the kernel ids whose bit (1u << id) is set in mask (default: all).
 * Each timed launch adds an event pair to its stream, so timing only the kernel of interest
 * keeps that overhead out of a timed region.  Forgets pending records. */
int pkv_timing_select(uint32_t mask);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
