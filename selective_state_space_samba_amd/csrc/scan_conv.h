// scan_conv.h -- the short causal convolution + SiLU alone (page 1 section 3.4, "Input
// Projection and Short Convolution"; causal, tap k multiplying x_{t-3+k}, as in the Samba
// Guide's Step 1): u_t = SiLU(conv_b + sum_k conv_w[k] x_{t-3+k}).  A full layer feeds u to
// its x_proj, whose outputs (dt, B, C) the scan then consumes together with x; the scan
// kernels recompute u from x on the fly, so this kernel is only needed for x_proj's input.
//
// It reads 2 B and writes 2 B per token.channel (bf16) and does ~10 VALU ops there, so it
// is HBM-bound and laid out for streaming:
//  * a thread owns one 16-byte vector of consecutive channels (8 for bf16, 4 for fp32) of
//    one sequence and a run of consecutive tokens; the 64 lanes of a wave read and write
//    64 consecutive vectors of a token row (1 KB);
//  * the three inputs before a run are re-read from the rows before it (or taken from the
//    incoming history at the sequence start), so runs are independent;
//  * the thread whose run ends at the sequence end writes the outgoing history (the last
//    three inputs, oldest first).
#pragma once

#include "scan_common.h"

namespace samba {

namespace conv {
constexpr int kThreads = 256;
constexpr int kMinRun = 64;  // tokens per thread (more when a sequence needs > 65535 runs)
constexpr int kGroup = 8;    // token rows requested together
}  // namespace conv

struct ConvArgs {
    int nseq;
    int seqlen;          // tokens per sequence (fixed length) or max_seqlen (packed)
    const int32_t *cu;   // packed offsets [nseq + 1] or nullptr
    int total;           // tokens in the packed arrays; offsets are clamped to it
    int D;
    int run;             // tokens per thread
    int nruns;           // runs per sequence (= ceil(seqlen / run), at least 1)
    const void *x;
    int ldx;             // x row pitch in elements (0: D, the contiguous layout)
    const float *conv_w, *conv_b;
    const void *conv0;
    // nullable: conv0 is a ring [nseq][3][D] whose slot (conv_head[s] + k) mod 3 holds
    // history entry k (oldest first); nullptr: entry k is in slot k
    const int32_t *conv_head;
    void *u;
    void *conv_final;
};

namespace conv {

template <class Io, int kVec>
__device__ inline void load_vec(const typename Io::T *p, float *f)
{
    using T = typename Io::T;
    if constexpr (kVec == 1) {
        f[0] = to_f32(p[0]);
    } else if constexpr (sizeof(T) == 2) {
        static_assert(kVec == 8, "bf16 vectors are 16 bytes");
        const uint4 w = *reinterpret_cast<const uint4 *>(p);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16lo(ws[i]);
            f[2 * i + 1] = bf16hi(ws[i]);
        }
    } else {
        static_assert(kVec == 4, "fp32 vectors are 16 bytes");
        const float4 w = *reinterpret_cast<const float4 *>(p);
        f[0] = w.x;
        f[1] = w.y;
        f[2] = w.z;
        f[3] = w.w;
    }
}

// Vector stores are non-temporal: u is streamed out and not read again by this kernel
// (measured: 4.99 -> 5.11 TB/s on the long prompt, the rate of a plain device copy).
template <class Io, int kVec>
__device__ inline void store_vec(typename Io::T *p, const float *f)
{
    using T = typename Io::T;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    if constexpr (kVec == 1) {
        Io::st(p, 0, f[0]);
    } else if constexpr (sizeof(T) == 2) {
        const u32x4 v = {pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
    } else {
        const f32x4 v = {f[0], f[1], f[2], f[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
    }
}

}  // namespace conv

// grid.x = nseq * nruns (sequence, run), grid.y = channel-vector blocks of 256.
template <class Io, int kVec>
__global__ __launch_bounds__(conv::kThreads) void conv_silu_kernel(ConvArgs a)
{
    using namespace conv;
    using T = typename Io::T;
    const int s = blockIdx.x / a.nruns;
    const int r = blockIdx.x - s * a.nruns;
    const int nvec = a.D / kVec;  // kVec divides D (checked at launch)
    const int g = blockIdx.y * kThreads + threadIdx.x;
    if (g >= nvec) return;  // no barriers: an early exit is safe
    const int c = g * kVec;
    const int D = a.D;
    const size_t ldx = a.ldx > 0 ? static_cast<size_t>(a.ldx) : static_cast<size_t>(D);

    size_t t0, t1;
    {
        if (a.cu != nullptr) {
            const int lo = min(max(a.cu[s], 0), a.total);
            const int hi = min(max(a.cu[s + 1], lo), a.total);
            t0 = static_cast<size_t>(lo);
            t1 = static_cast<size_t>(hi);
        } else {
            t0 = static_cast<size_t>(s) * static_cast<size_t>(a.seqlen);
            t1 = t0 + static_cast<size_t>(a.seqlen);
        }
    }
    const int L = static_cast<int>(t1 - t0);
    const int tb = r * a.run;
    if (tb >= L && r > 0) return;  // run 0 always runs: it passes the history of an empty sequence
    const int te = L - tb > a.run ? tb + a.run : L;

    const T *xs = static_cast<const T *>(a.x);
    T *us = static_cast<T *>(a.u);
    float w[kVec][kConvK], cb[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
        const float4 wv = *reinterpret_cast<const float4 *>(a.conv_w + static_cast<size_t>(c + i) * kConvK);
        w[i][0] = wv.x;
        w[i][1] = wv.y;
        w[i][2] = wv.z;
        w[i][3] = wv.w;
        cb[i] = a.conv_b ? a.conv_b[c + i] : 0.0f;
    }
    // win[k] = inputs of token t-3+k (k = 0, 1, 2) before token t.
    float win[3][kVec];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int tt = tb - 3 + k;
        if (tt >= 0) {
            load_vec<Io, kVec>(xs + (t0 + static_cast<size_t>(tt)) * ldx + c, win[k]);
        } else if (a.conv0 != nullptr) {
            const int slot = a.conv_head != nullptr ? ring_slot(a.conv_head[s], 3 + tt) : 3 + tt;
            load_vec<Io, kVec>(static_cast<const T *>(a.conv0) + (static_cast<size_t>(s) * 3 + slot) * D + c, win[k]);
        } else {
#pragma unroll
            for (int i = 0; i < kVec; ++i) win[k][i] = 0.0f;
        }
    }
    // One token: u from the window and the new inputs, then slide the window.
    auto token = [&](size_t row, const float *xv) {
        float uv[kVec];
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
            float pre = __builtin_fmaf(w[i][0], win[0][i], cb[i]);
            pre = __builtin_fmaf(w[i][1], win[1][i], pre);
            pre = __builtin_fmaf(w[i][2], win[2][i], pre);
            pre = __builtin_fmaf(w[i][3], xv[i], pre);
            uv[i] = silu(pre);
            win[0][i] = win[1][i];
            win[1][i] = win[2][i];
            win[2][i] = xv[i];
        }
        store_vec<Io, kVec>(us + row, uv);
    };
    // Groups of kGroup tokens: all of a group's rows are requested before any is used.
    int t = tb;
    for (; t + kGroup <= te; t += kGroup) {
        float xv[kGroup][kVec];
#pragma unroll
        for (int k = 0; k < kGroup; ++k)
            load_vec<Io, kVec>(xs + (t0 + static_cast<size_t>(t + k)) * ldx + c, xv[k]);
#pragma unroll
        for (int k = 0; k < kGroup; ++k) token((t0 + static_cast<size_t>(t + k)) * D + c, xv[k]);
    }
    for (; t < te; ++t) {
        float xv[kVec];
        load_vec<Io, kVec>(xs + (t0 + static_cast<size_t>(t)) * ldx + c, xv);
        token((t0 + static_cast<size_t>(t)) * D + c, xv);
    }
    if (te == L && a.conv_final != nullptr) {  // this run holds the sequence end
#pragma unroll
        for (int k = 0; k < 3; ++k)
            store_vec<Io, kVec>(static_cast<T *>(a.conv_final) + (static_cast<size_t>(s) * 3 + k) * D + c, win[k]);
    }
}

inline void launch_conv_silu(ConvArgs a, samba_dtype io, hipStream_t stream)
{
    const int elem = io == SAMBA_BF16 ? 2 : 4;
    const int vec = 16 / elem;
    const bool vectors = a.D % vec == 0;
    // Runs of at least kMinRun tokens, and no more than 65535 runs per sequence.
    const long long want = (static_cast<long long>(a.seqlen) + 65534) / 65535;
    a.run = static_cast<int>(want > conv::kMinRun ? want : conv::kMinRun);
    const long long nruns = (static_cast<long long>(a.seqlen) + a.run - 1) / a.run;
    a.nruns = static_cast<int>(nruns > 1 ? nruns : 1);
    const int nvec = vectors ? a.D / vec : a.D;
    const dim3 grid(static_cast<unsigned>(a.nseq) * static_cast<unsigned>(a.nruns),
                    (nvec + conv::kThreads - 1) / conv::kThreads);
    const dim3 block(conv::kThreads);
    if (io == SAMBA_BF16) {
        if (vectors)
            conv_silu_kernel<IoBf16, 8><<<grid, block, 0, stream>>>(a);
        else
            conv_silu_kernel<IoBf16, 1><<<grid, block, 0, stream>>>(a);
    } else {
        if (vectors)
            conv_silu_kernel<IoF32, 4><<<grid, block, 0, stream>>>(a);
        else
            conv_silu_kernel<IoF32, 1><<<grid, block, 0, stream>>>(a);
    }
}

}  // namespace samba
