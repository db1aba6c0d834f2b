// scan_lane.h -- one lane per (sequence, channel), sequential in time.
//
// Each lane keeps its channel's d_state fp32 states in registers and walks the
// sequence token by token (page 1 section 3.4, "The State Space Model Update (S6)":
// the recurrent form).  This kernel serves varlen and fixed-length prefill when
// batch * d_inner alone gives enough lanes to fill the GPU, and shapes the row kernels do
// not take.
//  * B_t and C_t are shared by every channel of a sequence and a workgroup holds channels
//    of one sequence, so they are read with scalar loads through the constant address space
//    (the kernel never writes them) and widened on the scalar unit: no vector-memory or VALU
//    work per state for them.
//  * x, dt and z are read kAhead tokens ahead into a small register ring, so a token's
//    loads have kAhead tokens of arithmetic to arrive.
#pragma once

#include "scan_common.h"

namespace samba {

namespace lane {

constexpr int kAhead = 4;  // tokens of x / dt / z in flight

template <class T>
using ConstPtr = const __attribute__((address_space(4))) T *;

// B_t and C_t (d_state = 16) as 32 uniform floats.
template <class Io>
__device__ inline void bc_row(const ScanArgs &a, size_t t, float *b, float *c)
{
    if constexpr (sizeof(typename Io::T) == 2) {
        const ConstPtr<uint32_t> pb = (ConstPtr<uint32_t>)(static_cast<const uint16_t *>(a.B) + t * kMaxState);
        const ConstPtr<uint32_t> pc = (ConstPtr<uint32_t>)(static_cast<const uint16_t *>(a.C) + t * kMaxState);
#pragma unroll
        for (int k = 0; k < kMaxState / 2; ++k) {
            const uint32_t wb = pb[k], wc = pc[k];
            b[2 * k] = bf16lo(wb);
            b[2 * k + 1] = bf16hi(wb);
            c[2 * k] = bf16lo(wc);
            c[2 * k + 1] = bf16hi(wc);
        }
    } else {
        const ConstPtr<float> pb = (ConstPtr<float>)(static_cast<const float *>(a.B) + t * kMaxState);
        const ConstPtr<float> pc = (ConstPtr<float>)(static_cast<const float *>(a.C) + t * kMaxState);
#pragma unroll
        for (int k = 0; k < kMaxState; ++k) {
            b[k] = pb[k];
            c[k] = pc[k];
        }
    }
}

}  // namespace lane

template <class Io, bool kFullN>
__global__ __launch_bounds__(256) void lane_scan_kernel(ScanArgs a)
{
    using namespace lane;
    using T = typename Io::T;
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
    const bool has_z = a.z != nullptr;
    const T *xs = static_cast<const T *>(a.x);
    const T *dts = static_cast<const T *>(a.dt);
    const T *zs = has_z ? static_cast<const T *>(a.z) : xs;

    // One token of the recurrence; B_t / C_t in b / c.
    auto step = [&](size_t t, float xv, float dtv, float zv, const float *b, const float *c) {
        float pre = __builtin_fmaf(w0, x0, cb);
        pre = __builtin_fmaf(w1, x1, pre);
        pre = __builtin_fmaf(w2, x2, pre);
        pre = __builtin_fmaf(w3, xv, pre);
        const float u = silu(pre);
        x0 = x1;
        x1 = x2;
        x2 = xv;
        // Delta in log2 units, then Delta * u
        const float lg = softplus_log2(dtv + bias);
        const float du = (lg * kLn2) * u;
        float acc = dsk * u;
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) {
            const float ab = hw_exp2(lg * Ad[n]);
            h[n] = __builtin_fmaf(ab, h[n], du * b[n]);
            acc = __builtin_fmaf(c[n], h[n], acc);
        }
        const float o = has_z ? acc * silu(zv) : acc;
        Io::st(a.out, t * D + d, o);
    };

    if constexpr (kFullN) {
        if (t1 <= t0) goto done;  // empty sequence: nothing to read
        // Token words kAhead tokens ahead (clamped re-loads past the end, never used).
        const size_t last = t1 - 1;
        T rx[kAhead], rd[kAhead], rz[kAhead];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
            const size_t ix = min(t0 + i, last) * D + d;
            rx[i] = xs[ix];
            rd[i] = dts[ix];
            rz[i] = zs[ix];
        }
        for (size_t tg = t0; tg < t1; tg += kAhead) {
            T cx[kAhead], cd[kAhead], cz[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) {
                cx[i] = rx[i];
                cd[i] = rd[i];
                cz[i] = rz[i];
                const size_t ix = min(tg + kAhead + i, last) * D + d;
                rx[i] = xs[ix];
                rd[i] = dts[ix];
                rz[i] = zs[ix];
            }
#pragma unroll
            for (int i = 0; i < kAhead; ++i) {
                const size_t t = tg + i;
                if (t < t1) {  // uniform: every lane of the workgroup is in the same sequence
                    float b[kMaxState], c[kMaxState];
                    bc_row<Io>(a, t, b, c);
                    step(t, to_f32(cx[i]), to_f32(cd[i]), to_f32(cz[i]), b, c);
                }
            }
        }
    } else {
        for (size_t t = t0; t < t1; ++t) {
            const size_t ix = t * D + d;
            float b[kMaxState], c[kMaxState];
#pragma unroll
            for (int n = 0; n < kMaxState; ++n) {
                const bool on = n < N;
                b[n] = on ? Io::ld(a.B, t * N + n) : 0.0f;
                c[n] = on ? Io::ld(a.C, t * N + n) : 0.0f;
            }
            step(t, Io::ld(a.x, ix), Io::ld(a.dt, ix), has_z ? Io::ld(a.z, ix) : 0.0f, b, c);
        }
    }

done:
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
