// Read probe: the HBM read rate that a plain kernel reaches on this device, as a
// reference beside the decode kernel's.  Paged decode is bound by reading the
// cache blocks back from memory (ithome article 10417389, section 3, and the
// glossary's "How paging works": the kernel fetches each block through the
// table), so its ceiling is a read stream, either sequential or of scattered
// tiles the size of one (block, KV head) tile of the pools.
//
// Work split: one wave64 per workgroup, as the decode kernel's workers.  The
// tiles to read, taken in list order, form rows of 1 KB (64 lanes x 16 bytes:
// one load instruction); the rows are cut into equal contiguous shares, one
// per wave.  A wave reads its share in batches of U rows, two batches deep: the
// next batch is issued before the current one is consumed, so at least U loads
// stay in flight, as in the decode kernel's load ring.  A tile holds whole
// rows, so the tile of a row is the same for all lanes and its id is a scalar
// load, which never waits behind the data loads.  A sequential read streams
// one contiguous region per wave.  Loads are non-temporal, as the decode
// kernel's; everything read is XOR-folded into one word per lane, stored at the
// end, so the loads cannot be dropped.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kProbeLanes = 64;
constexpr int kProbeUnroll = 8;
constexpr int kProbeRowShift = 6;        // 64 chunks of 16 bytes per row

typedef unsigned probe_u32x4_t __attribute__((ext_vector_type(4)));

template <bool IDS>
struct ProbeShare {
  const probe_u32x4_t* buf;
  const int64_t* tile_ids;
  int64_t num_buf_tiles, lo, hi;         // rows [lo, hi) of this wave; hi > lo
  int tile_shift;                        // log2 of 16-byte chunks per tile (>= 6 with ids)
  int lane;

  // row r of the tile list, lane's 16 bytes (zeros past the share; the address is
  // clamped to the share's last row, so no lane branches)
  __device__ __forceinline__ probe_u32x4_t load(int64_t r) const {
    const int64_t rr = r < hi ? r : hi - 1;
    int64_t chunk = (rr << kProbeRowShift) + lane;
    if constexpr (IDS) {
      const int64_t t = __builtin_amdgcn_readfirstlane(int(rr >> (tile_shift - kProbeRowShift)));
      int64_t id = tile_ids[t];
      if (id < 0 || id >= num_buf_tiles) id = 0;          // ids outside the buffer read tile 0
      chunk = (id << tile_shift) + (chunk & ((int64_t(1) << tile_shift) - 1));
    }
    const probe_u32x4_t v = __builtin_nontemporal_load(buf + chunk);
    return r < hi ? v : probe_u32x4_t{0u, 0u, 0u, 0u};
  }
};

__device__ __forceinline__ uint32_t fold(const probe_u32x4_t (&v)[kProbeUnroll]) {
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  return x;
}

template <bool IDS>
__global__ __launch_bounds__(kProbeLanes) void read_probe_kernel(
    const probe_u32x4_t* __restrict__ buf, int tile_shift, int64_t num_buf_tiles,
    const int64_t* __restrict__ tile_ids, int64_t rows, uint32_t* __restrict__ sink) {
  const int64_t W = gridDim.x, w = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t lo = rows * w / W, hi = rows * (w + 1) / W;
  uint32_t acc = 0;
  if (hi > lo) {
    const ProbeShare<IDS> sh{buf, tile_ids, num_buf_tiles, lo, hi, tile_shift, lane};
    probe_u32x4_t a[kProbeUnroll], b[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) a[u] = sh.load(lo + u);
    for (int64_t r = lo; r < hi; r += 2 * kProbeUnroll) {
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) b[u] = sh.load(r + kProbeUnroll + u);
      acc ^= fold(a);
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) a[u] = sh.load(r + 2 * kProbeUnroll + u);
      acc ^= fold(b);
    }
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
  if (tile_ids && shift < kProbeRowShift)
    return fail(PKV_E_INVAL, "tiles read through ids must hold at least 1024 bytes");
  if ((num_tiles << shift) & ((int64_t(1) << kProbeRowShift) - 1))
    return fail(PKV_E_INVAL, "num_tiles * tile_bytes must be a multiple of 1024");
  const int64_t rows = (num_tiles << shift) >> kProbeRowShift;
  const auto* b = static_cast<const probe_u32x4_t*>(buf);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (tile_ids)
    read_probe_kernel<true><<<dim3(unsigned(workgroups)), dim3(kProbeLanes), 0, s>>>(
        b, shift, buf_tiles, tile_ids, rows, sink);
  else
    read_probe_kernel<false><<<dim3(unsigned(workgroups)), dim3(kProbeLanes), 0, s>>>(
        b, shift, buf_tiles, nullptr, rows, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "read probe launch: %s", hipGetErrorString(e));
  return PKV_OK;
}
