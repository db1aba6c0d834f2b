// scan_lane.h -- one lane per (sequence, channel), sequential in time.
//
// Each lane keeps its channel's d_state fp32 states in registers and walks the
// sequence token by token (page 1 section 3.4, "The State Space Model Update (S6)":
// the recurrent form).  B_t and C_t are shared by every channel of a sequence, so within
// a workgroup (all lanes of one sequence) their loads are uniform.  This kernel serves
// the decode step (one token, state read and written in place), varlen and fixed-length
// prefill when batch * d_inner alone gives enough lanes to fill the GPU.
#pragma once

#include "scan_common.h"

namespace samba {

template <class Io, bool kFullN>
__global__ __launch_bounds__(256) void lane_scan_kernel(ScanArgs a)
{
    const int d = blockIdx.x * blockDim.x + threadIdx.x;
    const int s = blockIdx.y;
    if (d >= a.D) return;  // no barriers below: an early exit is safe
    const int D = a.D;
    const int N = kFullN ? kMaxState : a.N;

    size_t t0, t1;
    seq_range(a, s, t0, t1);

    float Ad[kMaxState], h[kMaxState];
    const size_t hbase = (static_cast<size_t>(s) * D + d) * N;
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) {
        const bool on = kFullN || n < N;
        Ad[n] = on ? a.A[static_cast<size_t>(d) * N + n] : 0.0f;
        h[n] = (on && a.h0 != nullptr) ? a.h0[hbase + n] : 0.0f;
    }
    const float w0 = a.conv_w[d * kConvK + 0], w1 = a.conv_w[d * kConvK + 1];
    const float w2 = a.conv_w[d * kConvK + 2], w3 = a.conv_w[d * kConvK + 3];
    const float cb = a.conv_b ? a.conv_b[d] : 0.0f;
    const float dsk = a.Dskip ? a.Dskip[d] : 0.0f;
    const float bias = a.dt_bias ? a.dt_bias[d] : 0.0f;
    const size_t cbase = static_cast<size_t>(s) * 3 * D + d;
    float x0 = 0.0f, x1 = 0.0f, x2 = 0.0f;  // x_{t-3}, x_{t-2}, x_{t-1}
    if (a.conv0 != nullptr) {
        x0 = Io::ld(a.conv0, cbase);
        x1 = Io::ld(a.conv0, cbase + D);
        x2 = Io::ld(a.conv0, cbase + 2 * static_cast<size_t>(D));
    }

    for (size_t t = t0; t < t1; ++t) {
        const size_t ix = t * D + d;
        const float xv = Io::ld(a.x, ix);
        // short convolution + SiLU
        float pre = __builtin_fmaf(w0, x0, cb);
        pre = __builtin_fmaf(w1, x1, pre);
        pre = __builtin_fmaf(w2, x2, pre);
        pre = __builtin_fmaf(w3, xv, pre);
        const float u = silu(pre);
        x0 = x1;
        x1 = x2;
        x2 = xv;
        // Delta in log2 units, then Delta * u
        const float lg = softplus_log2(Io::ld(a.dt, ix) + bias);
        const float du = (lg * kLn2) * u;
        float acc = dsk * u;
        const size_t ib = t * N;
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) {
            const bool on = kFullN || n < N;
            const float bn = on ? Io::ld(a.B, ib + n) : 0.0f;
            const float cn = on ? Io::ld(a.C, ib + n) : 0.0f;
            const float ab = hw_exp2(lg * Ad[n]);
            h[n] = __builtin_fmaf(ab, h[n], du * bn);
            acc = __builtin_fmaf(cn, h[n], acc);
        }
        const float o = (a.z != nullptr) ? acc * silu(Io::ld(a.z, ix)) : acc;
        Io::st(a.out, ix, o);
    }

    if (a.h_final != nullptr) {
#pragma unroll
        for (int n = 0; n < kMaxState; ++n)
            if (kFullN || n < N) a.h_final[hbase + n] = h[n];
    }
    if (a.conv_final != nullptr) {
        Io::st(a.conv_final, cbase, x0);
        Io::st(a.conv_final, cbase + D, x1);
        Io::st(a.conv_final, cbase + 2 * static_cast<size_t>(D), x2);
    }
}

inline void launch_lane_scan(const ScanArgs &a, samba_dtype io, hipStream_t stream)
{
    const dim3 block(256);
    const dim3 grid((a.D + 255) / 256, a.nseq);
    const bool full = a.N == kMaxState;
    if (io == SAMBA_BF16) {
        if (full)
            lane_scan_kernel<IoBf16, true><<<grid, block, 0, stream>>>(a);
        else
            lane_scan_kernel<IoBf16, false><<<grid, block, 0, stream>>>(a);
    } else {
        if (full)
            lane_scan_kernel<IoF32, true><<<grid, block, 0, stream>>>(a);
        else
            lane_scan_kernel<IoF32, false><<<grid, block, 0, stream>>>(a);
    }
}

}  // namespace samba
