// scan_decode.h -- one decode step for many resident sequences (d_state = 16).
//
// Generation advances every sequence by one token at constant cost: the fixed-size state
// is read, updated once and written back (page 1 section 5, generation throughput; the
// recurrence of section 3.4, "The State Space Model Update (S6)", with L = 1).  The step
// is bound by streaming the float32 state (2 x 64 bytes per sequence and channel), so
// the kernel is laid out for memory:
//  * a wave owns 64 consecutive channels of one sequence, whose states are one contiguous
//    4 KB block; it moves the block as four fully coalesced 1 KB rows of 16-byte vectors
//    (lane l, vector k: channel 16k + l/4, states 4(l%4)..4(l%4)+3), and A likewise.  (A
//    lane-per-channel layout, 64 B per lane, sustains about 30 % less bandwidth.)
//  * the per-channel front end (conv history, SiLU, softplus, gate) runs one lane per
//    channel on coalesced 2-byte rows; Delta and Delta*u reach the four lanes that hold a
//    channel's states by a cross-lane permute, the readout's partial sums are added across
//    those four lanes by DPP, and skip and gate terms return by a permute;
//  * the conv history is a ring of three slots per sequence: the step reads the three
//    slots from the head (the oldest) on and overwrites only the head slot with the new
//    input (144 bytes per sequence and channel per step in all); the next head goes to
//    head_out.
#pragma once

#include "scan_common.h"

namespace samba {

namespace dec {

constexpr int kQuadPerm1032 = 0xB1;  // quad_perm:[1,0,3,2]
constexpr int kQuadPerm2301 = 0x4E;  // quad_perm:[2,3,0,1]

template <int kCtrl>
__device__ inline float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, true));
}

// Value of v in lane src of the wave.
__device__ inline float from_lane(float v, int src)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

__device__ inline void widen4(const uint16_t *p, float *f)
{
    const uint2 w = *reinterpret_cast<const uint2 *>(p);
    f[0] = bf16lo(w.x);
    f[1] = bf16hi(w.x);
    f[2] = bf16lo(w.y);
    f[3] = bf16hi(w.y);
}
__device__ inline void widen4(const float *p, float *f)
{
    const float4 v = *reinterpret_cast<const float4 *>(p);
    f[0] = v.x;
    f[1] = v.y;
    f[2] = v.z;
    f[3] = v.w;
}

}  // namespace dec

template <class Io>
__global__ __launch_bounds__(256) void decode16_kernel(int D, int ldx, int ldbc, const typename Io::T *__restrict__ x,
                                                       const typename Io::T *__restrict__ dt,
                                                       const typename Io::T *__restrict__ Bm,
                                                       const typename Io::T *__restrict__ Cm,
                                                       const typename Io::T *__restrict__ z,
                                                       const float *__restrict__ A, const float *__restrict__ Dskip,
                                                       const float *__restrict__ dt_bias,
                                                       const float *__restrict__ conv_w,
                                                       const float *__restrict__ conv_b, float *__restrict__ h,
                                                       typename Io::T *__restrict__ conv,
                                                       const int32_t *__restrict__ head_in,
                                                       int32_t *__restrict__ head_out, typename Io::T *__restrict__ out)
{
    using namespace dec;
    using T = typename Io::T;
    constexpr int N = kMaxState;
    const int s = blockIdx.y;
    const int l = threadIdx.x & 63;
    const int c0 = blockIdx.x * 256 + (threadIdx.x & ~63);  // first channel of the wave
    if (c0 >= D) return;  // whole wave past the end; no barriers, so an early exit is safe

    // ---- front end, one lane per channel cf = c0 + l
    const int cf = c0 + l;
    const bool fok = cf < D;
    const int cfc = fok ? cf : D - 1;  // clamped for loads
    const size_t sdf = static_cast<size_t>(s) * D + cfc;
    const size_t sxf = static_cast<size_t>(s) * ldx + cfc;  // x and z may be column blocks of wider rows
    // ring slots of x_{t-3}, x_{t-2}, x_{t-1} (the head is the same for the whole wave)
    const int hd = __builtin_amdgcn_readfirstlane(head_in[s]);
    const size_t cbase = static_cast<size_t>(s) * 3 * D + cfc;
    const int k0 = ring_slot(hd, 0), k1 = ring_slot(hd, 1), k2 = ring_slot(hd, 2);
    const T h0 = conv[cbase + static_cast<size_t>(k0) * D], h1 = conv[cbase + static_cast<size_t>(k1) * D];
    const T h2 = conv[cbase + static_cast<size_t>(k2) * D];
    const T xr = x[sxf];
    const float dtv = to_f32(dt[sdf]);
    const float zv = z ? to_f32(z[sxf]) : 0.0f;
    const float4 w = *reinterpret_cast<const float4 *>(conv_w + static_cast<size_t>(cfc) * kConvK);
    const float cb = conv_b ? conv_b[cfc] : 0.0f;
    const float dsk = Dskip ? Dskip[cfc] : 0.0f;
    const float bias = dt_bias ? dt_bias[cfc] : 0.0f;

    // ---- state, A, B, C in the coalesced layout: vector k of lane l holds states
    // n0..n0+3 of channel ck = c0 + 16k + l/4
    const int n0 = 4 * (l & 3);
    const size_t hb = (static_cast<size_t>(s) * D + c0) * N;  // first state of the wave's block
    float hs[4][4], Av[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int ck = c0 + 16 * k + (l >> 2);
        const int ckc = ck < D ? ck : D - 1;
        const float4 hv = *reinterpret_cast<const float4 *>(h + hb + (static_cast<size_t>(ckc - c0) * N + n0));
        const float4 av = *reinterpret_cast<const float4 *>(A + static_cast<size_t>(ckc) * N + n0);
        hs[k][0] = hv.x; hs[k][1] = hv.y; hs[k][2] = hv.z; hs[k][3] = hv.w;
        Av[k][0] = av.x; Av[k][1] = av.y; Av[k][2] = av.z; Av[k][3] = av.w;
    }
    float Bv[4], Cv[4];
    widen4(Bm + static_cast<size_t>(s) * ldbc + n0, Bv);
    widen4(Cm + static_cast<size_t>(s) * ldbc + n0, Cv);

    // conv (tap k multiplies x_{t-3+k}) + SiLU, Delta (log2 units), skip and gate terms
    float pre = __builtin_fmaf(w.x, to_f32(h0), cb);
    pre = __builtin_fmaf(w.y, to_f32(h1), pre);
    pre = __builtin_fmaf(w.z, to_f32(h2), pre);
    pre = __builtin_fmaf(w.w, to_f32(xr), pre);
    const float u = silu(pre);
    const float lg = softplus_log2(dtv + bias);
    const float du = (lg * kLn2) * u;
    const float dskip = dsk * u;
    const float gate = z ? silu(zv) : 1.0f;
    if (fok) conv[cbase + static_cast<size_t>(k0) * D] = xr;  // the new input replaces the oldest
    if (head_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) head_out[s] = ring_slot(hd, 1);

    // ---- recurrence and partial readout over this lane's 4 states of 4 channels
    float part[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int src = 16 * k + (l >> 2);
        const float lgk = from_lane(lg, src), duk = from_lane(du, src);
        float acc = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float ab = hw_exp2(lgk * Av[k][v]);
            hs[k][v] = __builtin_fmaf(ab, hs[k][v], duk * Bv[v]);
            acc = __builtin_fmaf(Cv[v], hs[k][v], acc);
        }
        part[k] = acc;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int ck = c0 + 16 * k + (l >> 2);
        if (ck < D)
            *reinterpret_cast<float4 *>(h + hb + (static_cast<size_t>(ck - c0) * N + n0)) =
                make_float4(hs[k][0], hs[k][1], hs[k][2], hs[k][3]);
    }
    // sum over the 4 lanes of a channel (all four end with the channel's sum)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        part[k] += dpp<kQuadPerm1032>(part[k]);
        part[k] += dpp<kQuadPerm2301>(part[k]);
    }

    // ---- output: lane l finishes channel co = c0 + 16 (l%4) + l/4 (its sum is part[l%4])
    const int q = l & 3;
    const float y = q == 0 ? part[0] : q == 1 ? part[1] : q == 2 ? part[2] : part[3];
    const int src = 16 * q + (l >> 2);
    const float o = (y + from_lane(dskip, src)) * from_lane(gate, src);
    const int co = c0 + src;
    if (co < D) Io::st(out, static_cast<size_t>(s) * D + co, o);
}

inline void launch_decode16(const ScanArgs &a, samba_dtype io, hipStream_t stream)
{
    const dim3 block(256);
    const dim3 grid((a.D + 255) / 256, a.nseq);
    if (io == SAMBA_BF16) {
        using T = uint16_t;
        decode16_kernel<IoBf16><<<grid, block, 0, stream>>>(
            a.D, a.ldx > 0 ? a.ldx : a.D, a.ldbc > 0 ? a.ldbc : kMaxState, static_cast<const T *>(a.x), static_cast<const T *>(a.dt), static_cast<const T *>(a.B),
            static_cast<const T *>(a.C), static_cast<const T *>(a.z), a.A, a.Dskip, a.dt_bias, a.conv_w, a.conv_b,
            a.h_final, static_cast<T *>(a.conv_final), a.head_in, a.head_out, static_cast<T *>(a.out));
    } else {
        using T = float;
        decode16_kernel<IoF32><<<grid, block, 0, stream>>>(
            a.D, a.ldx > 0 ? a.ldx : a.D, a.ldbc > 0 ? a.ldbc : kMaxState, static_cast<const T *>(a.x), static_cast<const T *>(a.dt), static_cast<const T *>(a.B),
            static_cast<const T *>(a.C), static_cast<const T *>(a.z), a.A, a.Dskip, a.dt_bias, a.conv_w, a.conv_b,
            a.h_final, static_cast<T *>(a.conv_final), a.head_in, a.head_out, static_cast<T *>(a.out));
    }
}

}  // namespace samba
