// Measured fp32 matrix-core peak of the device the benchmark runs on.
//
// Every wave issues independent chains of v_mfma_f32_32x32x2_f32 (4096 flop
// each) on register operands only: no memory traffic, no vector-ALU work
// inside the timed loop.  The benchmark times one launch with events for the
// throughput; one wave per workgroup also reads the shader clock counter
// (s_memtime) and the 100 MHz real-time counter (s_memrealtime) around its
// loop, so the clock the peak was reached at can be reported beside it.
// Built as its own small library (libkia_peak.so): it is a measuring aid and
// no part of the K-interval attention path.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void kia_peak_kernel(float* out, unsigned long long* clk, int iters) {
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
    const float a = (float)threadIdx.x * 1e-3f, b = 1.0f + (float)blockIdx.x * 1e-7f;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 16; ++s)
            acc[s & 3] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[s & 3], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[c][r];
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
    if (threadIdx.x == 0) {
        clk[2 * (size_t)blockIdx.x] = t1 - t0;
        clk[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

extern "C" {

// Launch `grid` workgroups of 256 threads, each wave issuing 16 * iters
// matrix instructions.  out: grid * 256 floats; clk: 2 * grid uint64 (shader
// clock cycles and 100 MHz ticks of wave 0 of every workgroup).  Returns the
// hipError_t of the launch.
int kia_peak_mfma_f32(float* out, unsigned long long* clk, int iters, int grid, void* stream) {
    if (!out || !clk || iters < 1 || grid < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(kia_peak_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, out, clk, iters);
    return (int)hipGetLastError();
}

}  // extern "C"
