// Read probe: the HBM read rate that a plain kernel reaches on this device, as a
// reference beside the decode kernel's.  Paged decode is bound by reading the
// cache blocks back from memory (ithome article 10417389, section 3, and the
// glossary's "How paging works": the kernel fetches each block through the
// table), so its ceiling is a read stream, either sequential or of scattered
// tiles the size of one (block, KV head) tile of the pools.
//
// Work split: one wave64 per workgroup, as the decode kernel's workers.  The
// tiles to read, taken in list order as one run of 16-byte chunks, are cut
// into equal contiguous shares, one per wave; a wave reads its share 1 KB per
// load instruction (64 lanes x 16 bytes, consecutive), U instructions in
// flight, so a sequential read streams one contiguous region per wave.  Loads
// are non-temporal, as the decode kernel's; everything read is XOR-folded into
// one word per lane, stored at the end, so the loads cannot be dropped.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kProbeLanes = 64;
constexpr int kProbeUnroll = 16;

typedef unsigned probe_u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeLanes) void read_probe_kernel(
    const probe_u32x4_t* __restrict__ buf, int tile_shift, int64_t num_buf_tiles,
    const int64_t* __restrict__ tile_ids, int64_t num_tiles, uint32_t* __restrict__ sink) {
  const int64_t W = gridDim.x, w = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t chunks = num_tiles << tile_shift;
  const int64_t lo = chunks * w / W, hi = chunks * (w + 1) / W;   // this wave's share
  const int64_t in_tile = (int64_t(1) << tile_shift) - 1;
  uint32_t acc = 0;
  for (int64_t c0 = lo + lane; c0 < hi; c0 += kProbeUnroll * kProbeLanes) {
    probe_u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t c = c0 + u * kProbeLanes;
      if (c < hi) {
        const int64_t t = c >> tile_shift;
        int64_t id = tile_ids ? tile_ids[t] : t;
        if (id < 0 || id >= num_buf_tiles) id = 0;       // ids outside the buffer read tile 0
        v[u] = __builtin_nontemporal_load(buf + (id << tile_shift) + (c & in_tile));
      } else {
        v[u] = probe_u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[w * kProbeLanes + lane] = acc;
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_read_probe(const void* buf, size_t buf_bytes, int64_t tile_bytes,
                              const int64_t* tile_ids, int64_t num_tiles, uint32_t* sink,
                              int32_t workgroups, void* stream) {
  clear_error();
  if (!buf || !sink) return fail(PKV_E_INVAL, "NULL pointer");
  if ((reinterpret_cast<uintptr_t>(buf) | reinterpret_cast<uintptr_t>(sink)) & 15u)
    return fail(PKV_E_INVAL, "buf and sink must be 16-byte aligned");
  if (tile_bytes < 16 || (tile_bytes & (tile_bytes - 1)))
    return fail(PKV_E_INVAL, "tile_bytes %lld is not a power of two of at least 16",
                static_cast<long long>(tile_bytes));
  if (workgroups <= 0 || workgroups > (1 << 20))
    return fail(PKV_E_INVAL, "workgroups %d out of range", workgroups);
  const int64_t buf_tiles = int64_t(buf_bytes / size_t(tile_bytes));
  if (num_tiles < 0 || buf_tiles == 0) return fail(PKV_E_INVAL, "no tiles to read");
  if (!tile_ids && num_tiles > buf_tiles)
    return fail(PKV_E_INVAL, "%lld sequential tiles exceed the buffer's %lld",
                static_cast<long long>(num_tiles), static_cast<long long>(buf_tiles));
  if (num_tiles == 0) return PKV_OK;
  int shift = 0;
  while ((int64_t(16) << shift) < tile_bytes) ++shift;
  read_probe_kernel<<<dim3(unsigned(workgroups)), dim3(kProbeLanes), 0,
                      static_cast<hipStream_t>(stream)>>>(
      static_cast<const probe_u32x4_t*>(buf), shift, buf_tiles, tile_ids, num_tiles, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "read probe launch: %s", hipGetErrorString(e));
  return PKV_OK;
}
