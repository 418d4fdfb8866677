// Flat-span KV storage: one contiguous virtual range per sequence, backed by physical memory on demand.
//
// The alternative to a block table that "Contiguous vs Paged KV Cache on RDNA4" names (sections "Is
// paging the only way to fix KV cache fragmentation?" and "Why the single-user verdict flipped"):
// reserve a flat virtual range per sequence up front and commit physical pages into it as the sequence
// grows, so the attention kernel reads each sequence as one span and needs no table, while the card still
// commits only what the sequences hold.
//
// MI355X design: one virtual reservation per pool (keys, values) is cut into max_spans equal spans.  A
// span keeps the pools' documented block layout, so span s holds "virtual blocks" s * blocks_per_span ..
// (s + 1) * blocks_per_span - 1 of one large virtual pool, and the scatter kernel and the decode kernel's
// tiles work on it unchanged; decode only computes block ids instead of reading them.  Physical memory
// comes in chunks of chunk_bytes (a multiple of the device's allocation granularity), created with
// hipMemCreate and mapped with hipMemMap / hipMemSetAccess.  A released span's chunks are unmapped and
// kept for reuse, so a steady state maps and unmaps without creating or freeing memory.
#include <algorithm>
#include <mutex>
#include <numeric>
#include <vector>

#include "pkv_internal.h"

struct pkv_span_pool {
  int device = 0;
  int32_t max_spans = 0, blocks_per_span = 0, block_size = 0;
  size_t block_bytes = 0, span_bytes = 0, chunk_bytes = 0;
  void* va[2] = {nullptr, nullptr};   // keys, values
  std::vector<std::vector<hipMemGenericAllocationHandle_t>> mapped[2];   // per pool, per span: chunks in order
  std::vector<hipMemGenericAllocationHandle_t> spare;                    // unmapped chunks kept for reuse
  size_t created = 0;
  std::mutex mu;
};

namespace {

using pkv::PKV_SPAN_DEFAULT_CHUNK;

hipMemAllocationProp chunk_prop(int device) {
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

int esize_of(int dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16:
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

// A chunk for the mapping: a spare one, or a new one.  hipErrorOutOfMemory becomes PKV_ERR_OOM.
int take_chunk(pkv_span_pool* p, hipMemGenericAllocationHandle_t* h) {
  if (!p->spare.empty()) {
    *h = p->spare.back();
    p->spare.pop_back();
    return PKV_OK;
  }
  hipMemAllocationProp prop = chunk_prop(p->device);
  const hipError_t e = hipMemCreate(h, p->chunk_bytes, &prop, 0);
  if (e == hipErrorOutOfMemory) return PKV_ERR_OOM;
  if (e != hipSuccess) return PKV_ERR_HIP;
  ++p->created;
  return PKV_OK;
}

// Maps chunk index c of span s in pool k to handle h, read-write for the pool's device.
hipError_t map_chunk(pkv_span_pool* p, int k, int32_t s, size_t c, hipMemGenericAllocationHandle_t h) {
  char* at = static_cast<char*>(p->va[k]) + static_cast<size_t>(s) * p->span_bytes + c * p->chunk_bytes;
  hipError_t e = hipMemMap(at, p->chunk_bytes, 0, h, 0);
  if (e != hipSuccess) return e;
  hipMemAccessDesc acc = {};
  acc.location.type = hipMemLocationTypeDevice;
  acc.location.id = p->device;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  e = hipMemSetAccess(at, p->chunk_bytes, &acc, 1);
  if (e != hipSuccess) (void)hipMemUnmap(at, p->chunk_bytes);
  return e;
}

// Unmaps span s's chunks from index `keep` on, in both pools, and keeps them as spares.
int shrink_span(pkv_span_pool* p, int32_t s, size_t keep) {
  int status = PKV_OK;
  for (int k = 0; k < 2; ++k) {
    auto& m = p->mapped[k][s];
    while (m.size() > keep) {
      const size_t c = m.size() - 1;
      char* at = static_cast<char*>(p->va[k]) + static_cast<size_t>(s) * p->span_bytes + c * p->chunk_bytes;
      if (hipMemUnmap(at, p->chunk_bytes) != hipSuccess) status = PKV_ERR_HIP;
      p->spare.push_back(m.back());
      m.pop_back();
    }
  }
  return status;
}

void destroy_all(pkv_span_pool* p) {
  for (int32_t s = 0; s < p->max_spans; ++s) shrink_span(p, s, 0);
  for (auto h : p->spare) (void)hipMemRelease(h);
  p->spare.clear();
  for (int k = 0; k < 2; ++k)
    if (p->va[k]) (void)hipMemAddressFree(p->va[k], p->span_bytes * static_cast<size_t>(p->max_spans));
}

}  // namespace

extern "C" {

int pkv_span_pool_create(int32_t max_spans, int32_t max_tokens, int32_t n_kv_heads, int32_t head_dim,
                         int32_t block_size, int dtype, size_t chunk_bytes, pkv_span_pool** out) {
  if (!out || max_spans <= 0 || max_tokens <= 0 || n_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return PKV_ERR_INVALID;
  const int es = esize_of(dtype);
  if (!es || head_dim % (16 / es)) return PKV_ERR_INVALID;
  *out = nullptr;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return PKV_ERR_HIP;
  int vmm = 0;
  if (hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, device) != hipSuccess)
    return PKV_ERR_HIP;
  if (!vmm) return PKV_ERR_UNSUPPORTED;
  hipMemAllocationProp prop = chunk_prop(device);
  size_t gran = 0;
  if (hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum) != hipSuccess || !gran)
    return PKV_ERR_HIP;
  const size_t chunk = chunk_bytes ? chunk_bytes : PKV_SPAN_DEFAULT_CHUNK;
  if (chunk % gran) return PKV_ERR_INVALID;
  const size_t block_bytes = static_cast<size_t>(n_kv_heads) * head_dim * block_size * es;
  // a span is a whole number of chunks and of blocks
  const size_t unit = std::lcm(chunk, block_bytes);
  const size_t want = static_cast<size_t>((static_cast<int64_t>(max_tokens) + block_size - 1) / block_size) * block_bytes;
  const size_t span_bytes = (want + unit - 1) / unit * unit;
  const size_t bps = span_bytes / block_bytes;
  if (bps > (size_t{1} << 30) || bps * static_cast<size_t>(max_spans) >= (size_t{1} << 31)) return PKV_ERR_UNSUPPORTED;
  auto* p = new pkv_span_pool();
  p->device = device;
  p->max_spans = max_spans;
  p->blocks_per_span = static_cast<int32_t>(bps);
  p->block_size = block_size;
  p->block_bytes = block_bytes;
  p->span_bytes = span_bytes;
  p->chunk_bytes = chunk;
  for (int k = 0; k < 2; ++k) p->mapped[k].assign(max_spans, {});   // before any failure path walks them
  for (int k = 0; k < 2; ++k) {
    if (hipMemAddressReserve(&p->va[k], span_bytes * static_cast<size_t>(max_spans), chunk, nullptr, 0) != hipSuccess) {
      p->va[k] = nullptr;
      destroy_all(p);
      delete p;
      return PKV_ERR_OOM;
    }
  }
  *out = p;
  return PKV_OK;
}

void pkv_span_pool_destroy(pkv_span_pool* p) {
  if (!p) return;
  {
    std::lock_guard<std::mutex> g(p->mu);
    destroy_all(p);
  }
  delete p;
}

int pkv_span_reserve(pkv_span_pool* p, int32_t span, int32_t n_tokens) {
  if (!p || span < 0 || span >= p->max_spans || n_tokens < 0) return PKV_ERR_INVALID;
  std::lock_guard<std::mutex> g(p->mu);
  const size_t blocks = (static_cast<size_t>(n_tokens) + p->block_size - 1) / p->block_size;
  if (blocks > static_cast<size_t>(p->blocks_per_span)) return PKV_ERR_INVALID;
  const size_t need = (blocks * p->block_bytes + p->chunk_bytes - 1) / p->chunk_bytes;
  const size_t had = p->mapped[0][span].size();
  for (int k = 0; k < 2; ++k) {
    auto& m = p->mapped[k][span];
    while (m.size() < need) {
      hipMemGenericAllocationHandle_t h;
      int st = take_chunk(p, &h);
      if (st == PKV_OK && map_chunk(p, k, span, m.size(), h) != hipSuccess) {
        p->spare.push_back(h);
        st = PKV_ERR_HIP;
      }
      if (st != PKV_OK) {   // all or nothing: back to what the span had
        shrink_span(p, span, had);
        return st;
      }
      m.push_back(h);
    }
  }
  return PKV_OK;
}

int pkv_span_release(pkv_span_pool* p, int32_t span) {
  if (!p || span < 0 || span >= p->max_spans) return PKV_ERR_INVALID;
  std::lock_guard<std::mutex> g(p->mu);
  return shrink_span(p, span, 0);
}

int pkv_span_pool_trim(pkv_span_pool* p) {
  if (!p) return PKV_ERR_INVALID;
  std::lock_guard<std::mutex> g(p->mu);
  int status = PKV_OK;
  for (auto h : p->spare) {
    if (hipMemRelease(h) != hipSuccess) status = PKV_ERR_HIP;
    --p->created;
  }
  p->spare.clear();
  return status;
}

int pkv_span_pool_info(pkv_span_pool* p, pkv_span_info* out) {
  if (!p || !out) return PKV_ERR_INVALID;
  std::lock_guard<std::mutex> g(p->mu);
  out->k_base = p->va[0];
  out->v_base = p->va[1];
  out->blocks_per_span = p->blocks_per_span;
  out->num_blocks = p->blocks_per_span * p->max_spans;
  out->chunk_bytes = p->chunk_bytes;
  out->span_bytes = p->span_bytes;
  size_t mapped = 0;
  for (int k = 0; k < 2; ++k)
    for (const auto& m : p->mapped[k]) mapped += m.size();
  out->mapped_bytes = mapped * p->chunk_bytes;
  out->spare_bytes = p->spare.size() * p->chunk_bytes;
  return PKV_OK;
}

int32_t pkv_span_mapped_tokens(pkv_span_pool* p, int32_t span) {
  if (!p || span < 0 || span >= p->max_spans) return -1;
  std::lock_guard<std::mutex> g(p->mu);
  const size_t bytes = p->mapped[0][span].size() * p->chunk_bytes;
  const size_t blocks = std::min(bytes / p->block_bytes, static_cast<size_t>(p->blocks_per_span));
  return static_cast<int32_t>(blocks * p->block_size);
}

}  // extern "C"
