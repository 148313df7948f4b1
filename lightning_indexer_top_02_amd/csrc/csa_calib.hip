// Measurement aid, not part of the indexer's C ABI: a plain streaming read
// that calibrates what a read-only kernel reaches from HBM on this GPU (the
// practical ceiling of the bandwidth-bound decode key scan).  Built into its
// own library (libcsa_calib.so); only the benchmark loads it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int RS_THREADS = 256;
constexpr int RS_UNROLL = 16;    // 16-byte loads in flight per lane
constexpr int RS_GRID = 8192;

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Every 16-byte piece of buf[0, n16) is loaded once.  Workgroup g reads the
// contiguous g-th share of the buffer, RS_UNROLL pieces in flight per lane,
// each load instruction 4 KB of consecutive bytes (whole cache lines), with
// the non-temporal hint (streamed data that nothing reads again).  The
// loaded words are XOR-folded; a workgroup writes its fold to sink only if it
// equals a value the host never produces, so the loads cannot be elided and
// nothing else is written.  (Measured on MI355X: grid-stride 16-byte loads
// without the hint reach about 5.4 TB/s, contiguous shares 6.3 TB/s, with
// the hint 7.0-7.1 TB/s.)
__global__ __launch_bounds__(RS_THREADS) void csa_read_stream_kernel(const uint4* __restrict__ buf, size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t e0 = b0 + per < n16 ? b0 + per : n16;
  const u32x4* p = (const u32x4*)buf;
  uint32_t acc = 0u;
  size_t i = b0 + threadIdx.x;
  for (; i + (RS_UNROLL - 1) * RS_THREADS < e0; i += RS_UNROLL * RS_THREADS) {
    u32x4 v[RS_UNROLL];
#pragma unroll
    for (int j = 0; j < RS_UNROLL; ++j) v[j] = __builtin_nontemporal_load(&p[i + j * RS_THREADS]);
#pragma unroll
    for (int j = 0; j < RS_UNROLL; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  for (; i < e0; i += RS_THREADS) {
    const u32x4 v = __builtin_nontemporal_load(&p[i]);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from the 16-byte aligned device buffer
// `buf` on `stream`; sink must hold `grid` words (the return value of
// csa_calib_read_grid).  Returns 0, or a nonzero HIP error code.
extern "C" int csa_calib_read_grid(void) { return RS_GRID; }

extern "C" int csa_calib_read_stream(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes % 16 || (uintptr_t)buf % 16) return (int)hipErrorInvalidValue;
  csa_read_stream_kernel<<<csa_calib_read_grid(), RS_THREADS, 0, (hipStream_t)stream>>>((const uint4*)buf,
                                                                                      bytes / 16, sink);
  return (int)hipGetLastError();
}
