// Read-bandwidth calibration kernel (diagnostic; see include/pa_diag.h).
//
// Each wave64 streams whole tiles with 16-byte non-temporal loads (load i of a tile covers bytes
// [1024 i, 1024 i + 1024), lane l the 16 bytes at 16 l), in address order or in the order of a
// permutation -- the pattern of the paged kernels, which fetch one (block, head) tile at a time
// from scattered blocks. Every loaded word is folded into a running XOR that is stored only under
// a condition the data never meets, so no load can be removed.

#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_diag.h"

namespace {

template <int TILE_KB>
__global__ __launch_bounds__(256) void read_tiles_kernel(const uint8_t* __restrict__ buf,
                                                         const int32_t* __restrict__ order,
                                                         int num_tiles, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  uint32_t acc = 0;
  for (int i = wave; i < num_tiles; i += nwaves) {
    const int t = order != nullptr ? order[i] : i;
    const pa::u32x4* p = reinterpret_cast<const pa::u32x4*>(buf + static_cast<size_t>(t) * TILE_KB * 1024) + lane;
    pa::u32x4 v[TILE_KB];
#pragma unroll
    for (int k = 0; k < TILE_KB; ++k) v[k] = __builtin_nontemporal_load(p + 64 * k);
#pragma unroll
    for (int k = 0; k < TILE_KB; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (acc == 0x9e3779b9u) sink[(blockIdx.x * 256 + threadIdx.x) & 0xffff] = acc;
}

template <int TILE_KB>
hipError_t launch(const void* buf, const int32_t* order, int n, uint32_t* sink, hipStream_t st) {
  int waves = n < 256 * 32 ? n : 256 * 32;
  const int groups = (waves + 3) / 4;
  hipLaunchKernelGGL(read_tiles_kernel<TILE_KB>, dim3(groups), dim3(256), 0, st,
                     static_cast<const uint8_t*>(buf), order, n, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" int pa_diag_read_bandwidth(const void* buf, size_t buffer_tiles, const int32_t* tile_order,
                                      int num_tiles, int tile_bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || num_tiles <= 0 || tile_bytes <= 0 || tile_bytes % 1024 != 0 ||
      tile_bytes > (1 << 20))
    return PA_ERR_INVALID_ARG;
  if (tile_order == nullptr && buffer_tiles < static_cast<size_t>(num_tiles)) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (tile_bytes / 1024) {
    case 1: e = launch<1>(buf, tile_order, num_tiles, sink, st); break;
    case 2: e = launch<2>(buf, tile_order, num_tiles, sink, st); break;
    case 4: e = launch<4>(buf, tile_order, num_tiles, sink, st); break;
    case 8: e = launch<8>(buf, tile_order, num_tiles, sink, st); break;
    case 16: e = launch<16>(buf, tile_order, num_tiles, sink, st); break;
    default: return PA_ERR_UNSUPPORTED;
  }
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}
