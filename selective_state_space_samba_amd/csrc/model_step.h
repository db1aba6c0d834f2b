// model_step.h -- the kernels a whole Samba decode step adds around the layer cores (gfx950).
//
// Page "Samba: Simple Hybrid State Space Models for Efficient Unlimited Context Language
// Modeling" (paper-graph-ui summary), "The layer arrangement pattern": every Mamba, SWA and
// MLP layer is preceded by RMSNorm and followed by a residual skip connection.  The residual
// stream is kept in float32; RMSNorm writes the bfloat16 operand of the next projections.
#pragma once

#include "scan_common.h"

namespace samba {
namespace step {

// out[r][:] = x[r][:] / sqrt(mean(x[r][:]^2) + eps) * w[:], one workgroup of 256 threads per
// row; the sum of squares is accumulated in float32 per lane, then across the wave by lane
// shuffles and across the 4 waves through LDS (a fixed order, so the result is deterministic).
__global__ __launch_bounds__(256) void rmsnorm_kernel(int rows, int d, const float *__restrict__ x,
                                                      const float *__restrict__ w, float eps,
                                                      uint16_t *__restrict__ out)
{
    const int r = blockIdx.x;
    if (r >= rows) return;
    const float *xr = x + static_cast<size_t>(r) * d;
    float s = 0.f;
    for (int i = threadIdx.x; i < d; i += 256) s = __builtin_fmaf(xr[i], xr[i], s);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = __builtin_amdgcn_rsqf(tot / static_cast<float>(d) + eps);
    uint16_t *orow = out + static_cast<size_t>(r) * d;
    for (int i = threadIdx.x; i < d; i += 256)
        orow[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(xr[i] * inv * w[i]));
}

// The same with 16-byte accesses: thread t holds elements 8 (256 c + t) .. + 7 of the row for
// c < NCH in registers between the sum of squares and the scaling, so the row is read once
// (d a multiple of 8, at most 2048 NCH; x, w and out 16-byte aligned).  The per-thread sum
// runs over its elements in order, then the same wave and LDS steps: deterministic.
template <int NCH>
__global__ __launch_bounds__(256) void rmsnorm_vec_kernel(int rows, int d, const float *__restrict__ x,
                                                          const float *__restrict__ w, float eps,
                                                          uint16_t *__restrict__ out)
{
    const int r = blockIdx.x;
    if (r >= rows) return;
    const float *xr = x + static_cast<size_t>(r) * d;
    float v[NCH][8];
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int i = (c * 256 + threadIdx.x) * 8;
        if (i < d) {
            const float4 a = *reinterpret_cast<const float4 *>(xr + i);
            const float4 b = *reinterpret_cast<const float4 *>(xr + i + 4);
            v[c][0] = a.x, v[c][1] = a.y, v[c][2] = a.z, v[c][3] = a.w;
            v[c][4] = b.x, v[c][5] = b.y, v[c][6] = b.z, v[c][7] = b.w;
#pragma unroll
            for (int e = 0; e < 8; ++e) s = __builtin_fmaf(v[c][e], v[c][e], s);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = __builtin_amdgcn_rsqf(tot / static_cast<float>(d) + eps);
    uint16_t *orow = out + static_cast<size_t>(r) * d;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int i = (c * 256 + threadIdx.x) * 8;
        if (i < d) {
            const float4 a = *reinterpret_cast<const float4 *>(w + i);
            const float4 b = *reinterpret_cast<const float4 *>(w + i + 4);
            const float ws[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pk[e] = pack_bf16(v[c][2 * e] * inv * ws[2 * e], v[c][2 * e + 1] * inv * ws[2 * e + 1]);
            *reinterpret_cast<uint4 *>(orow + i) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
    }
}

// After a step the positions advance by one token (negative = inactive, kept) and the
// Mamba layers' conv-ring head moves to the next slot (every sequence: the Mamba layers
// advance inactive sequences too).  conv_head may be nullptr (a stack without Mamba layers).
__global__ __launch_bounds__(256) void advance_pos_kernel(int n, int32_t *pos, int32_t *conv_head)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    if (pos[i] >= 0) pos[i] += 1;
    if (conv_head != nullptr) conv_head[i] = ring_slot(conv_head[i], 1);
}

inline void launch_rmsnorm(int rows, int d, const float *x, const float *w, float eps, uint16_t *out,
                           hipStream_t s)
{
    if (rows <= 0) return;
    const auto a16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const int nch = (d + 2047) / 2048;
    if (d % 8 == 0 && nch <= 4 && a16(x) && a16(w) && a16(out)) {
        switch (nch) {
        case 1: hipLaunchKernelGGL(rmsnorm_vec_kernel<1>, dim3(rows), dim3(256), 0, s, rows, d, x, w, eps, out); return;
        case 2: hipLaunchKernelGGL(rmsnorm_vec_kernel<2>, dim3(rows), dim3(256), 0, s, rows, d, x, w, eps, out); return;
        case 3: hipLaunchKernelGGL(rmsnorm_vec_kernel<3>, dim3(rows), dim3(256), 0, s, rows, d, x, w, eps, out); return;
        default: hipLaunchKernelGGL(rmsnorm_vec_kernel<4>, dim3(rows), dim3(256), 0, s, rows, d, x, w, eps, out); return;
        }
    }
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, rows, d, x, w, eps, out);
}

inline void launch_advance(int n, int32_t *pos, int32_t *conv_head, hipStream_t s)
{
    if (n > 0) hipLaunchKernelGGL(advance_pos_kernel, dim3((n + 255) / 256), dim3(256), 0, s, n, pos, conv_head);
}

}  // namespace step
}  // namespace samba
