// Device probes for the benchmark (not part of the SSD ABI): the fp32 MFMA
// rate that a loop of independent v_mfma_f32_32x32x2f32 chains reaches on
// every SIMD of the chip, and the shader clock during that loop (the
// shader-clock counter against the fixed-rate real-time counter); and the
// lane-operation rates of fp32 multiply-adds and of exponentials.
#include <hip/hip_runtime.h>

#include <stdint.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;   // independent accumulator chains per wave

// Every wave runs `iters` groups of kChains MFMAs (4 waves per block, one per
// SIMD).  Lane 0 of wave 0 of block b writes its shader-clock and real-time
// counters at the start and end to ticks[4b .. 4b+3]; every lane writes its
// sum of the accumulators to sink so the loop is not removed.
__global__ __launch_bounds__(256) void k_mfma_loop(float *__restrict__ sink, uint64_t *__restrict__ ticks,
                                                   int iters)
{
    f32x16 acc[kChains];
    for (int c = 0; c < kChains; ++c)
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    const float a = 1e-3f * (float)(threadIdx.x & 7), b = 1e-3f;
    const bool rec = threadIdx.x == 0;
    uint64_t c0 = 0, r0 = 0;
    if (rec) {
        c0 = clock64();
        r0 = wall_clock64();
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
    for (int c = 0; c < kChains; ++c)
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
    if (rec) {
        const uint64_t c1 = clock64(), r1 = wall_clock64();
        ticks[4 * blockIdx.x + 0] = c0;
        ticks[4 * blockIdx.x + 1] = c1;
        ticks[4 * blockIdx.x + 2] = r0;
        ticks[4 * blockIdx.x + 3] = r1;
    }
}

// Every thread runs `iters` rounds of kVChains independent chains of one
// operation (MODE 0: multiply-add, MODE 1: base-2 exponential) and writes one
// float of their sum to sink[blockIdx.x * 256 + threadIdx.x].
constexpr int kVChains = 8;
template <int MODE>
__global__ __launch_bounds__(256) void k_valu_loop(float *__restrict__ sink, float c, float d, int iters)
{
    float x[kVChains];
#pragma unroll
    for (int i = 0; i < kVChains; ++i) x[i] = 1e-3f * (float)(threadIdx.x + i);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kVChains; ++i) x[i] = MODE == 0 ? __builtin_fmaf(x[i], c, d) : __builtin_amdgcn_exp2f(x[i]);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kVChains; ++i) s += x[i];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

extern "C" {

// Bytes of device memory probe_valu_loop needs for `blocks` blocks.
size_t probe_valu_loop_bytes(int blocks) { return (size_t)blocks * 256 * sizeof(float); }

// Launches k_valu_loop<mode> (0: fma, 1: exp) on `blocks` blocks of 256
// threads; lane operations per launch: blocks * 256 * iters *
// probe_valu_chains().  Returns 0 or -1.
int probe_valu_loop(void *buf, int blocks, int iters, int mode, void *stream)
{
    if (!buf || blocks < 1 || iters < 1 || mode < 0 || mode > 1) return -1;
    float *sink = static_cast<float *>(buf);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mode == 0)
        hipLaunchKernelGGL(k_valu_loop<0>, dim3(blocks), dim3(256), 0, st, sink, 0.999f, 1e-4f, iters);
    else
        hipLaunchKernelGGL(k_valu_loop<1>, dim3(blocks), dim3(256), 0, st, sink, 0.999f, 1e-4f, iters);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int probe_valu_chains(void) { return kVChains; }

// Bytes of device memory probe_mfma_loop needs for `blocks` blocks.
size_t probe_mfma_loop_bytes(int blocks) { return (size_t)blocks * (256 * sizeof(float) + 4 * sizeof(uint64_t)); }

// Launches the loop on `blocks` blocks of 256 threads; `buf` holds
// probe_mfma_loop_bytes(blocks) device bytes, the counters land at
// buf + blocks * 1024 bytes as [blocks][4] uint64.  FLOPs per launch:
// blocks * 4 waves * iters * kChains * 32*32*2*2.  Returns 0 or -1.
int probe_mfma_loop(void *buf, int blocks, int iters, void *stream)
{
    if (!buf || blocks < 1 || iters < 1) return -1;
    float *sink = static_cast<float *>(buf);
    uint64_t *ticks = reinterpret_cast<uint64_t *>(static_cast<char *>(buf) + (size_t)blocks * 256 * sizeof(float));
    hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), sink, ticks,
                       iters);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int probe_mfma_chains(void) { return kChains; }

// Rate of the real-time counter of the current device in kHz (0 if unknown).
int probe_wall_clock_khz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

}  // extern "C"
