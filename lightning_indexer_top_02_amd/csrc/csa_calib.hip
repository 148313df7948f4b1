// Measurement aid, not part of the indexer's C ABI: a plain streaming read
// that calibrates what a read-only kernel reaches from HBM on this GPU (the
// practical ceiling of the bandwidth-bound decode key scan).  Built into its
// own library (libcsa_calib.so); only the benchmark loads it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int RS_THREADS = 256;
constexpr int RS_UNROLL = 8;     // 16-byte loads in flight per lane

// Every 16-byte piece of buf[0, n16) is loaded once: lane-contiguous pieces,
// RS_UNROLL of them in flight per lane, grid-stride over the buffer.  The
// loaded words are XOR-folded; a workgroup writes its fold to sink only if it
// equals a value the host never produces, so the loads cannot be elided and
// nothing else is written.
__global__ __launch_bounds__(RS_THREADS) void csa_read_stream_kernel(const uint4* __restrict__ buf, size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * RS_THREADS;
  size_t i = (size_t)blockIdx.x * RS_THREADS + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (RS_UNROLL - 1) * stride < n16; i += RS_UNROLL * stride) {
    uint4 v[RS_UNROLL];
#pragma unroll
    for (int j = 0; j < RS_UNROLL; ++j) v[j] = buf[i + j * stride];
#pragma unroll
    for (int j = 0; j < RS_UNROLL; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from the 16-byte aligned device buffer
// `buf` on `stream`; sink must hold `grid` words (the return value of
// csa_calib_read_grid).  Returns 0, or a nonzero HIP error code.
extern "C" int csa_calib_read_grid(void) { return 256 * 16; }

extern "C" int csa_calib_read_stream(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes % 16 || (uintptr_t)buf % 16) return (int)hipErrorInvalidValue;
  csa_read_stream_kernel<<<csa_calib_read_grid(), RS_THREADS, 0, (hipStream_t)stream>>>((const uint4*)buf,
                                                                                      bytes / 16, sink);
  return (int)hipGetLastError();
}
