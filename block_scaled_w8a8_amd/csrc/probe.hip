// Measurement support: a kernel that keeps the fp8 matrix cores busy with nothing else, so the
// benchmark can state the MFMA throughput this GPU reaches in practice (at the clock it holds
// under load) beside the published dense fp8 peak. Every wave runs kChains independent
// accumulation chains of v_mfma_f32_16x16x128_f8f6f4 on register operands; no memory traffic
// but one store per lane at the end (which keeps the chains live).
#include "bfq_internal.h"
#include "device_common.h"

namespace bfq {

constexpr int kProbeChains = 8;         // independent MFMA chains per wave
constexpr int kProbeWaves = 8;          // waves per workgroup (two per SIMD)

__global__ __launch_bounds__(64 * kProbeWaves) void mfma_peak_kernel(int64_t iters, float* out) {
    const int lane = threadIdx.x & 63;
    // operands: small e4m3 codes that differ per lane (values are irrelevant to the timing)
    const int base = 0x30303030 + lane;
    const v8i a = {base, base + 1, base + 2, base + 3, base + 4, base + 5, base + 6, base + 7};
    const v8i b = {base + 7, base + 6, base + 5, base + 4, base + 3, base + 2, base + 1, base};
    v4f acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma_fp8_16x16x128_acc(a, b, acc[c]);
    }
    v4f s = acc[0];
#pragma unroll
    for (int c = 1; c < kProbeChains; ++c) s += acc[c];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s.x + s.y + s.z + s.w;
}

// grid: `blocks` workgroups of kProbeWaves waves; out holds blocks * 64 * kProbeWaves floats.
// flops = blocks * kProbeWaves * iters * kProbeChains * (2 * 16 * 16 * 128).
hipError_t launch_mfma_peak(int64_t blocks, int64_t iters, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(64 * kProbeWaves), 0, stream,
                       iters, out);
    return hipGetLastError();
}

int mfma_peak_threads_per_block() { return 64 * kProbeWaves; }
int mfma_peak_mfmas_per_wave_iter() { return kProbeChains; }

}  // namespace bfq
