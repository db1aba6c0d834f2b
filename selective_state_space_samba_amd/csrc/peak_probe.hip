// peak_probe.hip -- measures, on the GPU it runs on, the vector-ALU issue rates that bound
// the selective scan: fp32 FMA (VOP3 v_fma_f32 and VOP2 v_fmac_f32), the transcendental
// v_exp_f32, exponentials mixed 1:4 with independent FMAs in one wave and split between
// waves (does the transcendental unit run beside the FMAs?), the latency of a dependent
// FMA and of a dependent exponential (one chain per lane, one wave per SIMD), FMA and multiply
// with one operand in a scalar register (a wave-uniform value), and the shader clock during
// each run (s_memtime core-clock ticks against the constant-rate
// s_memrealtime counter).
//
// In the rate probes every lane runs 8 independent dependency chains, so neither one wave's
// latency nor the number of waves bounds the rate; the grid puts 8 waves on every SIMD.
// The chains' values stay finite (a contraction for the FMAs, 2^-|v| for the exponential).
// The instructions are written in inline assembly so that the compiler can neither fuse,
// pack nor remove them; they are ALU operations only (no memory access inside the asm).
//
// A measurement library for the benchmark, not part of the scan's C ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // loop body: kUnroll groups of 8 chains

enum Kind {
    kFma = 0, kExp = 1, kMix = 2, kFmac = 3, kMixWaves = 4, kFmaLat = 5, kExpLat = 6,
    kAddDpp = 7, kMulBcast = 8, kCndmask = 9, kMul = 10, kFmaSgpr = 11, kMulSgpr = 12
};

__device__ inline void fma8(float (&v)[8], float m, float c)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(v[i]) : "v"(m), "v"(c));
}
__device__ inline void fmac8(float (&v)[8], float m, float c)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(v[i]) : "v"(m), "v"(c));
}
// Cross-lane forms used by the scan kernels (each chain reads a register last written 8
// instructions earlier, beyond the 2 wait states a DPP read of a fresh VALU result needs).
__device__ inline void add_dpp8(float (&v)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i)
        asm volatile("v_add_f32_dpp %0, %0, %0 row_shl:1 row_mask:0xf bank_mask:0xf bound_ctrl:1" : "+v"(v[i]));
}
__device__ inline void mul_bcast8(float (&v)[8], float m)
{
#pragma unroll
    for (int i = 0; i < 8; ++i)
        asm volatile("v_mul_f32_dpp %0, %0, %1 row_newbcast:1 row_mask:0xf bank_mask:0xf bound_ctrl:1" : "+v"(v[i]) : "v"(m));
}
__device__ inline void cndmask8(float (&v)[8], float o)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("v_cndmask_b32_e64 %0, %0, %1, s[0:1]" : "+v"(v[i]) : "v"(o) : "s0", "s1");
}
__device__ inline void mul8(float (&v)[8], float m)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("v_mul_f32_e32 %0, %1, %0" : "+v"(v[i]) : "v"(m));
}
// The same with the multiplier in a scalar register.
__device__ inline void fma_s8(float (&v)[8], float m, float c)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(v[i]) : "s"(m), "v"(c));
}
__device__ inline void mul_s8(float (&v)[8], float m)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("v_mul_f32_e32 %0, %1, %0" : "+v"(v[i]) : "s"(m));
}
__device__ inline void exp8(float (&v)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("v_exp_f32 %0, -|%0|" : "+v"(v[i]));
}

template <int kKind>
__global__ __launch_bounds__(512) void probe_kernel(int iters, float seed, float *sink, uint64_t *stamps)
{
    float v[8], e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = seed + 0.01f * static_cast<float>(i + (threadIdx.x & 7));
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = v[i] + 0.5f;
    // kMixWaves (8-wave workgroups): half the waves run exponentials, half FMAs.  Waves w
    // and w ^ 1, and w and w ^ 4, always differ, so each SIMD gets one of each kind whether
    // the waves of a workgroup are dealt to the 4 SIMDs round-robin or two at a time.
    const int wv = threadIdx.x >> 6;
    const bool exp_wave = ((wv ^ (wv >> 2)) & 1) == 0;
    const float m = 0.999f, c = 0.001f;
    __syncthreads();
    uint64_t c0 = 0, w0 = 0;
    if (threadIdx.x == 0) {
        c0 = clock64();
        w0 = wall_clock64();
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (kKind == kFma) fma8(v, m, c);
            if (kKind == kFmac) fmac8(v, m, c);
            if (kKind == kExp) exp8(v);
            if (kKind == kMix) {
                // 8 exponentials and 32 FMAs (1 : 4) on independent registers
                exp8(e);
                fma8(v, m, c);
                fma8(v, m, c);
                fma8(v, m, c);
                fma8(v, m, c);
            }
            if (kKind == kMixWaves) {
                if (exp_wave)
                    exp8(e);
                else {
                    fma8(v, m, c);
                    fma8(v, m, c);
                    fma8(v, m, c);
                    fma8(v, m, c);
                }
            }
            if (kKind == kAddDpp) add_dpp8(v);
            if (kKind == kMulBcast) mul_bcast8(v, m);
            if (kKind == kCndmask) cndmask8(v, c);
            if (kKind == kMul) mul8(v, m);
            if (kKind == kFmaSgpr) fma_s8(v, m, c);
            if (kKind == kMulSgpr) mul_s8(v, m);
            if (kKind == kFmaLat) {
#pragma unroll
                for (int i = 0; i < 8; ++i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(v[0]) : "v"(m), "v"(c));
            }
            if (kKind == kExpLat) {
#pragma unroll
                for (int i = 0; i < 8; ++i) asm volatile("v_exp_f32 %0, -|%0|" : "+v"(v[0]));
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint64_t c1 = clock64(), w1 = wall_clock64();
        stamps[2 * blockIdx.x] = c1 - c0;
        stamps[2 * blockIdx.x + 1] = w1 - w0;
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i] + e[i];
    if (s == 12345.678f) sink[threadIdx.x] = s;  // keeps the chains live; never true in practice
}

}  // namespace

extern "C" {

// Runs probe `kind` over `workgroups` workgroups of 256 threads for `iters` loop trips,
// synchronously on the current device's null stream:
//   0 v_fma_f32, 3 v_fmac_f32, 1 v_exp_f32 (8 independent chains per lane);
//   2 one v_exp_f32 per four v_fma_f32 on independent registers, in every wave;
//   4 the same 1 : 4 mix split between waves (workgroups of 512 threads: on every SIMD one
//     wave of exponentials beside one of FMAs);
//   5 one dependent v_fma_f32 chain per lane; 6 one dependent v_exp_f32 chain per lane
//     (use one workgroup of 64 threads per SIMD for these two);
//   7 v_add_f32 with a DPP row_shl source, 8 v_mul_f32 with a DPP row_newbcast source,
//   9 v_cndmask_b32 (VOP3, SGPR-pair mask), 10 v_mul_f32 (VOP2), 11 v_fma_f32 and 12
//   v_mul_f32 with the multiplier in a scalar register: 8 chains per lane.
// Returns 0 on success.  Outputs:
//   out[0] seconds of the launch (HIP events)
//   out[1] lane-instructions executed (an exponential counts as one)
//   out[2] of them exponentials
//   out[3] median shader clock over the workgroups in GHz (s_memtime ticks / real time)
int samba_probe_rates(int kind, int workgroups, int iters, double *out)
{
    if (kind < 0 || kind > 12 || workgroups < 1 || iters < 1 || out == nullptr) return 1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 2;
    int wall_khz = 0;
    if (hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || wall_khz <= 0) return 2;
    float *sink = nullptr;
    uint64_t *stamps = nullptr;
    if (hipMalloc(&sink, 512 * sizeof(float)) != hipSuccess) return 2;  // one float per thread of the largest workgroup
    if (hipMalloc(&stamps, static_cast<size_t>(workgroups) * 2 * sizeof(uint64_t)) != hipSuccess) {
        (void)hipFree(sink);
        return 2;
    }
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    auto launch = [&](int n) {
        switch (kind) {
        case kFma: probe_kernel<kFma><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        case kExp: probe_kernel<kExp><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        case kMix: probe_kernel<kMix><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        case kMixWaves: probe_kernel<kMixWaves><<<workgroups, 512>>>(n, 0.5f, sink, stamps); break;
        case kFmaLat: probe_kernel<kFmaLat><<<workgroups, 64>>>(n, 0.5f, sink, stamps); break;
        case kExpLat: probe_kernel<kExpLat><<<workgroups, 64>>>(n, 0.5f, sink, stamps); break;
        case kAddDpp: probe_kernel<kAddDpp><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        case kMulBcast: probe_kernel<kMulBcast><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        case kCndmask: probe_kernel<kCndmask><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        case kMul: probe_kernel<kMul><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        case kFmaSgpr: probe_kernel<kFmaSgpr><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        case kMulSgpr: probe_kernel<kMulSgpr><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        default: probe_kernel<kFmac><<<workgroups, kThreads>>>(n, 0.5f, sink, stamps); break;
        }
    };
    launch(std::max(1, iters / 8));  // warm-up (clock ramp, code load)
    (void)hipEventRecord(e0, nullptr);
    launch(iters);
    (void)hipEventRecord(e1, nullptr);
    int rc = hipEventSynchronize(e1) == hipSuccess ? 0 : 2;
    float ms = 0.0f;
    if (rc == 0 && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) rc = 2;
    std::vector<uint64_t> st(static_cast<size_t>(workgroups) * 2);
    if (rc == 0 && hipMemcpy(st.data(), stamps, st.size() * sizeof(uint64_t), hipMemcpyDeviceToHost) != hipSuccess)
        rc = 2;
    if (rc == 0) {
        const bool lat = kind == kFmaLat || kind == kExpLat;
        const double lanes = static_cast<double>(workgroups) * (lat ? 64 : kind == kMixWaves ? 512 : kThreads);
        double per_iter = kUnroll * 8.0, exps = 0.0;
        if (kind == kExp || kind == kExpLat) exps = per_iter;
        if (kind == kMix) {
            per_iter = kUnroll * 40.0;
            exps = kUnroll * 8.0;
        }
        if (kind == kMixWaves) {  // half the lanes run 8 exponentials, half 32 FMAs per unit
            per_iter = kUnroll * 20.0;
            exps = kUnroll * 4.0;
        }
        std::vector<double> ghz;
        for (int b = 0; b < workgroups; ++b) {
            const double wall_s = static_cast<double>(st[2 * b + 1]) / (wall_khz * 1e3);
            if (wall_s > 0) ghz.push_back(static_cast<double>(st[2 * b]) / wall_s / 1e9);
        }
        std::sort(ghz.begin(), ghz.end());
        out[0] = ms * 1e-3;
        out[1] = lanes * iters * per_iter;
        out[2] = lanes * iters * exps;
        out[3] = ghz.empty() ? 0.0 : ghz[ghz.size() / 2];
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(sink);
    (void)hipFree(stamps);
    return rc;
}

}  // extern "C"
