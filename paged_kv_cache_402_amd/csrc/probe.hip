// Read-bandwidth probe for gfx950: what plain 16-byte vector reads of HBM reach on this
// device, in the access patterns of the decode kernel. It measures the achievable ceiling
// that the attention kernels are compared with (reads never reach the nominal 8 TB/s); it is
// not part of the attention path and no page defines it.
//
// Each 256-lane workgroup reads tiles_per_group tiles of tile_bytes contiguous bytes each:
// tile i of the list starts at byte tile_ids[i] * tile_bytes of the buffer. The group's tile
// ids are staged in LDS first (as the decode kernel keeps a partition's block ids at hand), then
// its lanes sweep the tiles' 16-byte vectors in order, eight loads in flight per lane. The
// loaded words are folded into one value per lane that is stored only if it equals a
// caller-given sentinel, so no load can be dropped and almost nothing is written. The loads
// take either the default cache policy or the non-temporal one that the attention kernels use
// for KV rows.
#include "common.h"
#include "launch.h"

namespace pkv {

constexpr int kProbeMaxTiles = 1024;   // tiles per workgroup (ids staged in LDS)
constexpr int kProbeInFlight = 8;      // 16-byte loads in flight per lane

template <bool NT>
__global__ __launch_bounds__(256) void read_probe_kernel(ProbeArgs a) {
  __shared__ int s_ids[kProbeMaxTiles];
  const int t0 = blockIdx.x * a.tiles_per_group;
  const int nt = min(a.tiles_per_group, a.num_tiles - t0);
  for (int i = threadIdx.x; i < nt; i += 256) {
    const int id = a.tile_ids[t0 + i];
    s_ids[i] = (unsigned)id < (unsigned)a.num_tile_slots ? id : -1;   // -1: outside the buffer
  }
  __syncthreads();
  const int shift = a.tile_log2 - 4;                 // log2 of 16-byte vectors per tile
  const int64_t total = (int64_t)nt << shift;
  uint32_t x = 0;
  for (int64_t i0 = threadIdx.x; i0 < total; i0 += 256 * kProbeInFlight) {
    u32x4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) {
      const int64_t i = i0 + u * 256;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (i < total) {
        const int id = s_ids[i >> shift];
        if (id >= 0) {
          const unsigned char* p =
              a.buf + ((size_t)id << a.tile_log2) + ((size_t)(i & ((1 << shift) - 1)) << 4);
          v[u] = NT ? load16_stream(p) : load16(p);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (x == a.sentinel) a.sink[0] = x;
}

hipError_t launch_read_probe(const ProbeArgs& a, hipStream_t stream) {
  const int groups = (a.num_tiles + a.tiles_per_group - 1) / a.tiles_per_group;
  if (groups == 0) return hipSuccess;
  if (a.nontemporal)
    hipLaunchKernelGGL(read_probe_kernel<true>, dim3(groups), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(read_probe_kernel<false>, dim3(groups), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
