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
//  * x, dt and z are read kAhead tokens ahead into two register banks that take turns, so a
//    token's loads have kAhead tokens of arithmetic to arrive and no register is copied;
//    B and C are read one token ahead.
//  * token rows are addressed through buffer resources rebased once per group of tokens,
//    so the per-token address arithmetic is gone from the vector ALU and rows past the
//    sequence end read as 0 without a clamp.
#pragma once

#include "scan_common.h"

namespace samba {

namespace lane {

constexpr int kAhead = 4;  // tokens of x / dt / z in flight

template <class T>
using ConstPtr = const __attribute__((address_space(4))) T *;

// B_t and C_t (d_state = 16) as raw 32-bit words: 8 + 8 for bf16, 16 + 16 for fp32.
template <class Io>
struct BcWords {
    static constexpr int kWords = kMaxState * static_cast<int>(sizeof(typename Io::T)) / 4;
    uint32_t b[kWords], c[kWords];

    __device__ inline void load(const ScanArgs &a, size_t t)
    {
        using T = typename Io::T;
        const ConstPtr<uint32_t> pb = (ConstPtr<uint32_t>)(static_cast<const T *>(a.B) + t * kMaxState);
        const ConstPtr<uint32_t> pc = (ConstPtr<uint32_t>)(static_cast<const T *>(a.C) + t * kMaxState);
#pragma unroll
        for (int k = 0; k < kWords; ++k) {
            b[k] = pb[k];
            c[k] = pc[k];
        }
    }

    // Makes the loaded words available here (the wait for them goes here, not at the load).
    __device__ inline void settle()
    {
#pragma unroll
        for (int k = 0; k < kWords; ++k) asm volatile("" : "+s"(b[k]), "+s"(c[k]));
    }

    // Widened to 16 + 16 uniform floats.
    __device__ inline void widen(float *fb, float *fc) const
    {
#pragma unroll
        for (int k = 0; k < kWords; ++k) {
            if constexpr (kWords == kMaxState / 2) {
                fb[2 * k] = bf16lo(b[k]);
                fb[2 * k + 1] = bf16hi(b[k]);
                fc[2 * k] = bf16lo(c[k]);
                fc[2 * k + 1] = bf16hi(c[k]);
            } else {
                fb[k] = __uint_as_float(b[k]);
                fc[k] = __uint_as_float(c[k]);
            }
        }
    }
};

}  // namespace lane

// kUIn: x holds u = SiLU(conv(x)) already (the conv, its parameters and the history are
// not used).
template <class Io, bool kFullN, bool kUIn>
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
    const float w0 = kUIn ? 0.0f : a.conv_w[d * kConvK + 0], w1 = kUIn ? 0.0f : a.conv_w[d * kConvK + 1];
    const float w2 = kUIn ? 0.0f : a.conv_w[d * kConvK + 2], w3 = kUIn ? 0.0f : a.conv_w[d * kConvK + 3];
    const float cb = (!kUIn && a.conv_b) ? a.conv_b[d] : 0.0f;
    const float dsk = a.Dskip ? a.Dskip[d] : 0.0f;
    const float bias = a.dt_bias ? a.dt_bias[d] : 0.0f;
    const size_t cbase = static_cast<size_t>(s) * 3 * D + d;
    // History entry k (oldest first) lives in slot k, or in ring slot (head + k) mod 3 when
    // the decode passes a ring head.
    const int hd = a.head_in != nullptr ? a.head_in[s] : 0;
    const size_t e0 = cbase + static_cast<size_t>(ring_slot(hd, 0)) * D;
    const size_t e1 = cbase + static_cast<size_t>(ring_slot(hd, 1)) * D;
    const size_t e2 = cbase + static_cast<size_t>(ring_slot(hd, 2)) * D;
    float x0 = 0.0f, x1 = 0.0f, x2 = 0.0f;  // x_{t-3}, x_{t-2}, x_{t-1}
    if (!kUIn && a.conv0 != nullptr) {
        x0 = Io::ld(a.conv0, e0);
        x1 = Io::ld(a.conv0, e1);
        x2 = Io::ld(a.conv0, e2);
    }
    const bool has_z = a.z != nullptr;
    const T *xs = static_cast<const T *>(a.x);
    const T *dts = static_cast<const T *>(a.dt);
    const T *zs = has_z ? static_cast<const T *>(a.z) : xs;

    // One token of the recurrence; B_t / C_t in b / c.
    auto step = [&](float xv, float dtv, float zv, const float *b, const float *c) -> float {
        float u;
        if constexpr (kUIn) {
            u = xv;
        } else {
            float pre = __builtin_fmaf(w0, x0, cb);
            pre = __builtin_fmaf(w1, x1, pre);
            pre = __builtin_fmaf(w2, x2, pre);
            pre = __builtin_fmaf(w3, xv, pre);
            u = silu(pre);
            x0 = x1;
            x1 = x2;
            x2 = xv;
        }
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
        return has_z ? acc * silu(zv) : acc;
    };

    if constexpr (kFullN) {
        if (t1 <= t0) goto done;  // empty sequence: nothing to read
        // Token rows are addressed through buffer resources rebased on each group of kAhead
        // tokens and sized to the rows the group touches (at most 2 kAhead, none past the
        // sequence end): row i of the group is at the constant lane offset vo[i], loads past
        // the end return 0 and are never used, and nothing is recomputed per token.
        const uint32_t row = static_cast<uint32_t>(D) * sizeof(T);
        uint32_t vo[2 * kAhead];
#pragma unroll
        for (int i = 0; i < 2 * kAhead; ++i) vo[i] = static_cast<uint32_t>(d) * sizeof(T) + i * row;
        auto group_rsrc = [&](const void *p, size_t tg) {
            const size_t rows = min(t1 - tg, static_cast<size_t>(2 * kAhead));
            return make_rsrc(static_cast<const char *>(p) + tg * row, static_cast<uint32_t>(rows * row));
        };
        // x / dt / z words kAhead tokens ahead in two register banks that take turns (a group
        // reads one bank while the next group's words arrive in the other: no copies), B / C
        // words one token ahead.
        struct Bank {
            T x[kAhead], dt[kAhead], z[kAhead];
        };
        auto fill = [&](Bank &k, size_t tg, int first) {  // rows first .. first+kAhead-1 of group tg
            const Rsrc gx = group_rsrc(xs, tg), gd = group_rsrc(dts, tg), gz = group_rsrc(zs, tg);
#pragma unroll
            for (int i = 0; i < kAhead; ++i) {
                buf_ld(gx, vo[first + i], k.x[i]);
                buf_ld(gd, vo[first + i], k.dt[i]);
                buf_ld(gz, vo[first + i], k.z[i]);
            }
        };
        const size_t last = t1 - 1;
        BcWords<Io> nw;
        nw.load(a, t0);
        auto token = [&](size_t t, T xr, T dr, T zr, Rsrc go, uint32_t voff) {
            BcWords<Io> cw = nw;
            if constexpr (BcWords<Io>::kWords == kMaxState / 2) cw.settle();  // wait here for the words loaded a token ago
            nw.load(a, min(t + 1, last));
            float b[kMaxState], c[kMaxState];
            cw.widen(b, c);
            buf_st(go, voff, step(to_f32(xr), to_f32(dr), to_f32(zr), b, c), static_cast<T *>(nullptr));
        };
        // kAhead tokens of group tg from bank k (only the first n when n < kAhead).
        auto run = [&](const Bank &k, size_t tg, int n) {
            const Rsrc go = group_rsrc(a.out, tg);
#pragma unroll
            for (int i = 0; i < kAhead; ++i)
                if (i < n) token(tg + i, k.x[i], k.dt[i], k.z[i], go, vo[i]);
        };
        Bank b0, b1;
        fill(b0, t0, 0);
        // Pairs of whole groups: straight-line code, no per-token branch.
        size_t tg = t0;
        for (; tg + 2 * kAhead <= t1; tg += 2 * kAhead) {
            fill(b1, tg, kAhead);
            run(b0, tg, kAhead);
            fill(b0, tg + kAhead, kAhead);
            run(b1, tg + kAhead, kAhead);
        }
        // The last t1 - tg < 2 kAhead tokens; rows tg .. tg+kAhead-1 are in b0.
        if (tg + kAhead <= t1) {
            fill(b1, tg, kAhead);
            run(b0, tg, kAhead);
            run(b1, tg + kAhead, static_cast<int>(t1 - tg - kAhead));
        } else if (tg < t1) {
            run(b0, tg, static_cast<int>(t1 - tg));
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
            Io::st(a.out, ix, step(Io::ld(a.x, ix), Io::ld(a.dt, ix), has_z ? Io::ld(a.z, ix) : 0.0f, b, c));
        }
    }

done:
    if (a.h_final != nullptr) {
#pragma unroll
        for (int n = 0; n < kMaxState; ++n)
            if (kFullN || n < N) a.h_final[hbase + n] = h[n];
    }
    if (!kUIn && a.conv_final != nullptr) {
        if (a.head_in != nullptr) {
            // ring after one token: the new head is the old head + 1, so the entries
            // (oldest first) go to slots head + 1, head + 2 and head
            Io::st(a.conv_final, e1, x0);
            Io::st(a.conv_final, e2, x1);
            Io::st(a.conv_final, e0, x2);
            if (a.head_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) a.head_out[s] = ring_slot(hd, 1);
        } else {
            Io::st(a.conv_final, cbase, x0);
            Io::st(a.conv_final, cbase + D, x1);
            Io::st(a.conv_final, cbase + 2 * static_cast<size_t>(D), x2);
        }
    }
}

inline void launch_lane_scan(const ScanArgs &a, samba_dtype io, hipStream_t stream)
{
    const dim3 block(256);
    const dim3 grid((a.D + 255) / 256, a.nseq);
    const bool full = a.N == kMaxState;
#define SAMBA_LANE(IO, FULL, UIN) lane_scan_kernel<IO, FULL, UIN><<<grid, block, 0, stream>>>(a)
    if (io == SAMBA_BF16) {
        if (a.u_in) {
            if (full) SAMBA_LANE(IoBf16, true, true); else SAMBA_LANE(IoBf16, false, true);
        } else {
            if (full) SAMBA_LANE(IoBf16, true, false); else SAMBA_LANE(IoBf16, false, false);
        }
    } else {
        if (a.u_in) {
            if (full) SAMBA_LANE(IoF32, true, true); else SAMBA_LANE(IoF32, false, true);
        } else {
            if (full) SAMBA_LANE(IoF32, true, false); else SAMBA_LANE(IoF32, false, false);
        }
    }
#undef SAMBA_LANE
}

}  // namespace samba
