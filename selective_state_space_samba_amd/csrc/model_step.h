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

// Positions of the sequences advance by one token after a step (negative = inactive, kept).
__global__ __launch_bounds__(256) void advance_pos_kernel(int n, int32_t *pos)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n && pos[i] >= 0) pos[i] += 1;
}

inline void launch_rmsnorm(int rows, int d, const float *x, const float *w, float eps, uint16_t *out,
                           hipStream_t s)
{
    if (rows > 0) hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, rows, d, x, w, eps, out);
}

inline void launch_advance(int n, int32_t *pos, hipStream_t s)
{
    if (n > 0) hipLaunchKernelGGL(advance_pos_kernel, dim3((n + 255) / 256), dim3(256), 0, s, n, pos);
}

}  // namespace step
}  // namespace samba
