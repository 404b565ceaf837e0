// Calibration kernel: a read-only stream at the rate the stage kernels' load
// path can reach. Each work group reads a contiguous run of 16 KB stages with
// the same direct global-to-LDS loads (non-temporal, three stages in flight in
// a four-slot LDS ring) and discards them; bench reports this rate beside the
// HBM peak.
#include "device_common.h"
#include "internal.h"

namespace dpn {

constexpr int kProbeStage = 16384;      // bytes per stage
constexpr int kProbeStages = 64;        // stages per work group (1 MB)


__global__ void __launch_bounds__(256) k_read_probe(const unsigned char* __restrict__ buf, int64_t nstages) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * kProbeStage];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t s0 = (int64_t)blockIdx.x * kProbeStages;
  const int nst = (int)min<int64_t>(kProbeStages, nstages - s0);
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  auto dma = [&](int st) {
    if (st >= nst) return;
    const unsigned char* src = buf + (s0 + st) * kProbeStage + (wv * 4) * 1024 + lane * 16;
    const uint32_t dst = base + (uint32_t)((st & 3) * kProbeStage + wv * 4 * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16_stream(src + j * 1024, dst + j * 1024);
  };
  dma(0);
  dma(1);
  dma(2);
  for (int st = 0; st < nst; ++st) {
    wait_after<4>(min(2, nst - 1 - st));
    block_barrier();
    dma(st + 3);
  }
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, hipStream_t s) {
  const int64_t nstages = bytes / kProbeStage;
  const int64_t blocks = (nstages + kProbeStages - 1) / kProbeStages;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)blocks), dim3(256), 0, s, (const unsigned char*)buf, nstages);
  return hipGetLastError();
}

}  // namespace dpn
