// Streaming-read probe: how fast this GPU's HBM delivers a read-only stream to waves shaped like the
// decode kernel's (single-wave workgroups, 16 bytes per lane per load), with nothing computed on the
// data.  It gives the measured read ceiling that the decode kernel's bandwidth is set beside, next to
// the 8 TB/s of the data sheet.  Not part of the decode path.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ inline u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Wave w reads `iters` batches of NL loads; each load is 64 lanes x 16 bytes = 1 KiB.  Two batches are
// in flight: the next batch is issued before the current one is consumed.  RANDOM: each 4 KiB chunk of
// the buffer is visited once, in an order scattered over the whole buffer (an odd multiplier mod a
// power of two is a permutation), as paged blocks are; otherwise the wave reads its own contiguous span.
template <int NL, bool NT, bool RANDOM>
__global__ __launch_bounds__(64) void read_probe_kernel(const u32x4* buf, int64_t iters, int64_t nchunks,
                                                        unsigned* sink) {
  const int lane = threadIdx.x;
  const int64_t w = blockIdx.x;
  const int64_t base = w * iters * NL;   // this wave's first 1 KiB load
  auto addr = [&](int64_t k) -> const u32x4* {   // load k of the wave (global index base + k)
    const int64_t g = base + k;
    if constexpr (RANDOM) {
      const int64_t chunk = ((g >> 2) * 0x9E3779B1ll) & (nchunks - 1);   // nchunks: a power of two
      return buf + chunk * 256 + (g & 3) * 64 + lane;
    } else {
      return buf + g * 64 + lane;
    }
  };
  u32x4 acc = {0u, 0u, 0u, 0u}, a[NL], b[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) a[j] = load16<NT>(addr(j));
  for (int64_t i = 0; i < iters; i += 2) {
    const bool more = i + 1 < iters;
#pragma unroll
    for (int j = 0; j < NL; ++j) b[j] = load16<NT>(addr(more ? (i + 1) * NL + j : j));
#pragma unroll
    for (int j = 0; j < NL; ++j) acc ^= a[j];
    const bool more2 = i + 2 < iters;
#pragma unroll
    for (int j = 0; j < NL; ++j) a[j] = load16<NT>(addr(more2 ? (i + 2) * NL + j : j));
    if (more) {
#pragma unroll
      for (int j = 0; j < NL; ++j) acc ^= b[j];
    }
  }
  // keeps every load live; the values are never checked
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B1u && lane == 0) sink[w & 1023] = acc.x;
}

template <int NL, bool NT>
const void* probe_ptr(bool random) {
  return random ? reinterpret_cast<const void*>(&read_probe_kernel<NL, NT, true>)
                : reinterpret_cast<const void*>(&read_probe_kernel<NL, NT, false>);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_read_probe(const void* buf, size_t bytes, int32_t waves_per_cu, int32_t loads_per_batch,
                              int mode, uint32_t* sink, size_t* bytes_read, void* stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) || waves_per_cu < 1 || waves_per_cu > 32 ||
      (mode & ~3))
    return PKV_ERR_INVALID;
  const bool nt = (mode & 1) != 0, random = (mode & 2) != 0;
  const void* fn = nullptr;
  switch (loads_per_batch) {
    case 4: fn = nt ? probe_ptr<4, true>(random) : probe_ptr<4, false>(random); break;
    case 8: fn = nt ? probe_ptr<8, true>(random) : probe_ptr<8, false>(random); break;
    case 16: fn = nt ? probe_ptr<16, true>(random) : probe_ptr<16, false>(random); break;
    default: return PKV_ERR_UNSUPPORTED;
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return PKV_ERR_HIP;
  const int64_t grid = static_cast<int64_t>(cus) * waves_per_cu;
  const int64_t per_batch = grid * loads_per_batch * 1024;   // bytes one batch of every wave reads
  int64_t iters = static_cast<int64_t>(bytes) / per_batch;
  // random chunks: the largest power-of-two chunk count within the buffer, and no more than that read
  int64_t nchunks = 1;
  while (nchunks * 2 * 4096 <= static_cast<int64_t>(bytes)) nchunks *= 2;
  if (random) iters = nchunks * 4096 / per_batch;
  if (iters < 1) return PKV_ERR_INVALID;
  if (bytes_read) *bytes_read = static_cast<size_t>(iters * per_batch);
  const void* b = buf;
  int64_t it = iters;
  void* args[] = {&b, &it, &nchunks, &sink};   // (each entry points at one kernel argument)
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(64), args, 0,
                         static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}
