// scan_decode.h -- one decode step for many resident sequences (d_state = 16).
//
// Generation advances every sequence by one token at constant cost: the fixed-size state
// is read, updated once and written back (page 1 section 5, generation throughput; the
// recurrence of section 3.4, "The State Space Model Update (S6)", with L = 1).  The step
// is bound by streaming the float32 state (2 x 64 bytes per sequence and channel), so
// the kernel is laid out for memory: one lane per (sequence, channel), its 16 states
// moved as four 16-byte vectors (a wave covers 4 KB contiguous), A likewise, the token
// inputs as coalesced 2-byte rows, and B_t / C_t -- shared by the whole workgroup -- as
// wave-uniform scalar loads widened on the scalar unit.  The conv history is shifted in
// place (oldest first).
#pragma once

#include "scan_common.h"

namespace samba {

template <class Io>
__global__ __launch_bounds__(256) void decode16_kernel(int D, const typename Io::T *__restrict__ x,
                                                       const typename Io::T *__restrict__ dt,
                                                       const typename Io::T *__restrict__ Bm,
                                                       const typename Io::T *__restrict__ Cm,
                                                       const typename Io::T *__restrict__ z,
                                                       const float *__restrict__ A, const float *__restrict__ Dskip,
                                                       const float *__restrict__ dt_bias,
                                                       const float *__restrict__ conv_w,
                                                       const float *__restrict__ conv_b, float *__restrict__ h,
                                                       typename Io::T *__restrict__ conv, typename Io::T *__restrict__ out)
{
    using T = typename Io::T;
    constexpr int N = kMaxState;
    const int s = blockIdx.y;
    const int d = blockIdx.x * blockDim.x + threadIdx.x;

    // B_t and C_t of sequence s: uniform across the workgroup.
    float Bv[N], Cv[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        Bv[n] = to_f32(Bm[static_cast<size_t>(s) * N + n]);
        Cv[n] = to_f32(Cm[static_cast<size_t>(s) * N + n]);
    }
    if (d >= D) return;  // no barriers: an early exit is safe

    const size_t sd = static_cast<size_t>(s) * D + d;
    float hs[N], Ad[N];
    const float4 *hp = reinterpret_cast<const float4 *>(h + sd * N);
    const float4 *ap = reinterpret_cast<const float4 *>(A + static_cast<size_t>(d) * N);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        const float4 hv = hp[k], av = ap[k];
        hs[4 * k] = hv.x; hs[4 * k + 1] = hv.y; hs[4 * k + 2] = hv.z; hs[4 * k + 3] = hv.w;
        Ad[4 * k] = av.x; Ad[4 * k + 1] = av.y; Ad[4 * k + 2] = av.z; Ad[4 * k + 3] = av.w;
    }
    const float4 w = *reinterpret_cast<const float4 *>(conv_w + static_cast<size_t>(d) * kConvK);
    const float cb = conv_b ? conv_b[d] : 0.0f;
    const float dsk = Dskip ? Dskip[d] : 0.0f;
    const float bias = dt_bias ? dt_bias[d] : 0.0f;
    const size_t cbase = static_cast<size_t>(s) * 3 * D + d;
    const T c0 = conv[cbase], c1 = conv[cbase + D], c2 = conv[cbase + 2 * static_cast<size_t>(D)];
    const T xr = x[sd];
    const float xv = to_f32(xr);
    const float dtv = to_f32(dt[sd]);
    const float zv = z ? to_f32(z[sd]) : 0.0f;

    // conv (tap k multiplies x_{t-3+k}) + SiLU, Delta (log2 units), recurrence, readout
    float pre = __builtin_fmaf(w.x, to_f32(c0), cb);
    pre = __builtin_fmaf(w.y, to_f32(c1), pre);
    pre = __builtin_fmaf(w.z, to_f32(c2), pre);
    pre = __builtin_fmaf(w.w, xv, pre);
    const float u = silu(pre);
    const float lg = softplus_log2(dtv + bias);
    const float du = (lg * kLn2) * u;
    float y = dsk * u;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float ab = hw_exp2(lg * Ad[n]);
        hs[n] = __builtin_fmaf(ab, hs[n], du * Bv[n]);
        y = __builtin_fmaf(Cv[n], hs[n], y);
    }
    const float o = z ? y * silu(zv) : y;

    float4 *hw = reinterpret_cast<float4 *>(h + sd * N);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) hw[k] = make_float4(hs[4 * k], hs[4 * k + 1], hs[4 * k + 2], hs[4 * k + 3]);
    conv[cbase] = c1;
    conv[cbase + D] = c2;
    conv[cbase + 2 * static_cast<size_t>(D)] = xr;
    Io::st(out, sd, o);
}

inline void launch_decode16(const ScanArgs &a, samba_dtype io, hipStream_t stream)
{
    const dim3 block(256);
    const dim3 grid((a.D + 255) / 256, a.nseq);
    if (io == SAMBA_BF16) {
        using T = uint16_t;
        decode16_kernel<IoBf16><<<grid, block, 0, stream>>>(
            a.D, static_cast<const T *>(a.x), static_cast<const T *>(a.dt), static_cast<const T *>(a.B),
            static_cast<const T *>(a.C), static_cast<const T *>(a.z), a.A, a.Dskip, a.dt_bias, a.conv_w, a.conv_b,
            a.h_final, static_cast<T *>(a.conv_final), static_cast<T *>(a.out));
    } else {
        using T = float;
        decode16_kernel<IoF32><<<grid, block, 0, stream>>>(
            a.D, static_cast<const T *>(a.x), static_cast<const T *>(a.dt), static_cast<const T *>(a.B),
            static_cast<const T *>(a.C), static_cast<const T *>(a.z), a.A, a.Dskip, a.dt_bias, a.conv_w, a.conv_b,
            a.h_final, static_cast<T *>(a.conv_final), static_cast<T *>(a.out));
    }
}

}  // namespace samba
