// scan_bwd.h -- gradients of the selective-scan layer core (training).
//
// Reverse-mode differentiation of the recurrence of page 1 section 3.4 ("Input Projection
// and Short Convolution" ... "Gated Output"): for the loss sum(dout . out) + dh_final .
// h_final + dconv_final . conv_final, with G_t[n] = dLoss/dh_t[n],
//   gy = dout SiLU(z),  dz = dout y SiLU'(z),  G_t = gy C_t + Abar_{t+1} G_{t+1},
//   dC_t[n] += gy h_t[n],  dB_t[n] += G Delta u,  dA[n] += G Abar h_{t-1} Delta,
//   dDelta = sum_n G (A Abar h_{t-1} + u B),  du = gy D + Delta sum_n G B,
//   ddt = dDelta sigmoid(dt + b),  dpre = du SiLU'(pre),
//   dx_{t-3+k} += w_k dpre,  dconv_w[k] += dpre x_{t-3+k},  dconv_b += dpre.
//
// Parallel in time: the sequence is cut into chunks of kChunk tokens and every (sequence,
// chunk, channel) gets a lane (one lane per channel, the 16 states in registers, as in the
// lane prefill kernel), so a training batch of 4 x 4096 tokens x 4096 channels gives 1M
// lanes.  Both recurrences are linear, so a chunk only needs two carries:
//   1. local pass (one lane per chunk, one sweep in time order): the chunk's state from a
//      zero start, H, its decay sum S = sum_t Delta_t log2(e) (the chunk maps h to
//      exp2(A S) h + H), and its adjoint from a zero end, E (maps R to exp2(A S) R + E),
//      accumulated forward as a sum of running products of the decay factors;
//   2. carry pass (one lane per sequence, channel and state, sequential over chunks): the
//      true state entering each chunk and the true adjoint entering it from the right, the
//      gradient of h0 falls out at the end;
//   3. full pass (one lane per group of chunks): the forward recomputed from the true start
//      kSub tokens at a time (two checkpoints per chunk in LDS), then the reverse with
//      every per-token gradient; dB / dC (sums over channels) are reduced over the wave's
//      64 channels through LDS and written as per-wave partials; dA, dD, dbias as
//      per-group partials; the conv-output gradient dpre goes to a float32 workspace;
//   4. conv pass: dx (the conv transposed over dpre), dconv0, dconv_w / dconv_b partials;
//   5. reductions of the partials.
#pragma once

#include "scan_common.h"

namespace samba {

namespace bwd {

constexpr int kChunk = 16;  // tokens per time chunk
constexpr int kSub = 4;     // tokens recomputed at a time in the full pass
constexpr int kNSub = kChunk / kSub;
constexpr int kGroup = 4;   // consecutive chunks per lane in the full pass
constexpr int kSplit = 32;  // row splits of the parameter reductions
constexpr int kLanes = 64;  // one wave per workgroup: 64 consecutive channels
constexpr int kRun = 64;    // tokens per thread in the conv pass
constexpr int kPar = 18;    // per-chunk parameter partials: dA[16], dD, ddt_bias
constexpr int kConvPar = 5; // per-run conv partials: dconv_w[4], dconv_b
constexpr int kBC = 2 * kMaxState;  // per-token dB[16], dC[16]
constexpr int kTilePitch = kBC + 1;  // LDS tile pitch (floats): conflict-free columns

template <class T>
using ConstPtr = const __attribute__((address_space(4))) T *;

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

}  // namespace bwd

struct BwdArgs {
    int nseq, seqlen;   // seqlen: tokens per sequence (fixed) or max_seqlen (packed)
    const int32_t *cu;  // packed offsets or nullptr
    int total;          // tokens in the packed arrays (packed) / nseq * seqlen
    int D, N;
    int nchunk;         // chunks per sequence slot = ceil(seqlen / kChunk)
    int nrun;           // conv-pass runs per sequence slot = ceil(seqlen / kRun)
    int nwave;          // channel waves = ceil(D / 64)
    int ngroup;         // chunk groups per sequence slot = ceil(nchunk / kGroup)
    const void *x, *dt, *B, *C, *z;
    const float *A, *Dskip, *dt_bias, *conv_w, *conv_b;
    const float *h0;
    const void *conv0;
    const void *dout;
    const float *dh_final;
    const void *dconv_final;
    void *dx, *ddt, *dB, *dC, *dz;
    float *dA, *dD, *ddt_bias, *dconv_w, *dconv_b, *dh0;
    void *dconv0;
    // workspace
    float *hck;   // [nseq][nchunk][D][16]  local end state -> true state entering the chunk
    float *eck;   // [nseq][nchunk][D][16]  local adjoint carry -> adjoint entering from the right (the full
                  //                          pass reads it at the last chunk of each group only)
    float *lsum;  // [nseq][nchunk][D]      sum of Delta log2(e) over the chunk
    float *dpre;  // [total][D]             gradient of the conv output before SiLU
    float *ppar;  // [nseq][ngroup][D][kPar]
    float *pbc;   // [total][nwave][kBC]
    float *pconv; // [nseq][nrun][D][kConvPar]
    float *par2;  // [kSplit][D][kPar]       per-split sums of ppar
    float *conv2; // [kSplit][D][kConvPar]   per-split sums of pconv
};

namespace bwd {

__device__ inline void seq_bounds(const BwdArgs &a, int s, size_t &t0, size_t &t1)
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

__device__ inline float sigmoid(float v) { return hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

// B_t or C_t row as 16 uniform floats (zeros past N).
template <class Io, bool kFullN>
__device__ inline void row16(const void *p, size_t t, int N, float *f)
{
    using T = typename Io::T;
    if constexpr (kFullN) {
        if constexpr (sizeof(T) == 2) {
            const ConstPtr<uint32_t> q = (ConstPtr<uint32_t>)(static_cast<const T *>(p) + t * kMaxState);
#pragma unroll
            for (int k = 0; k < kMaxState / 2; ++k) {
                const uint32_t w = q[k];
                f[2 * k] = bf16lo(w);
                f[2 * k + 1] = bf16hi(w);
            }
        } else {
            const ConstPtr<float> q = (ConstPtr<float>)(static_cast<const float *>(p) + t * kMaxState);
#pragma unroll
            for (int k = 0; k < kMaxState; ++k) f[k] = q[k];
        }
    } else {
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) f[n] = n < N ? Io::ld(p, t * N + n) : 0.0f;
    }
}

// Per-lane constants of a channel.
struct Chan {
    float A[kMaxState];
    float w0, w1, w2, w3, cb, dsk, bias;
};

__device__ inline void load_chan(const BwdArgs &a, int dc, Chan &ch)
{
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) ch.A[n] = n < a.N ? a.A[static_cast<size_t>(dc) * a.N + n] : 0.0f;
    const float4 w = *reinterpret_cast<const float4 *>(a.conv_w + static_cast<size_t>(dc) * kConvK);
    ch.w0 = w.x;
    ch.w1 = w.y;
    ch.w2 = w.z;
    ch.w3 = w.w;
    ch.cb = a.conv_b ? a.conv_b[dc] : 0.0f;
    ch.dsk = a.Dskip ? a.Dskip[dc] : 0.0f;
    ch.bias = a.dt_bias ? a.dt_bias[dc] : 0.0f;
}

// Input x of token tt of the sequence starting at t0 (tt may be -3..-1: the history).
template <class Io>
__device__ inline float x_at(const BwdArgs &a, int s, size_t t0, int tt, int dc)
{
    if (tt >= 0) return Io::ld(a.x, (t0 + static_cast<size_t>(tt)) * a.D + dc);
    if (a.conv0 == nullptr) return 0.0f;
    return Io::ld(a.conv0, (static_cast<size_t>(s) * 3 + static_cast<size_t>(3 + tt)) * a.D + dc);
}

// Front end of one token: pre-activation, u = SiLU(pre), a = dt + b, lg = softplus(a) log2 e.
struct Front {
    float pre, u, a, lg;
};

__device__ inline void front(const Chan &ch, float xm3, float xm2, float xm1, float xt, float dtv, Front &f)
{
    float pre = __builtin_fmaf(ch.w0, xm3, ch.cb);
    pre = __builtin_fmaf(ch.w1, xm2, pre);
    pre = __builtin_fmaf(ch.w2, xm1, pre);
    pre = __builtin_fmaf(ch.w3, xt, pre);
    f.pre = pre;
    f.u = silu(pre);
    f.a = dtv + ch.bias;
    f.lg = softplus_log2(f.a);
}

// gy = dout SiLU(z) (or dout without a gate).
__device__ inline float gate_grad(float g, bool has_z, float zv)
{
    return has_z ? g * (zv * sigmoid(zv)) : g;
}

}  // namespace bwd

// ---------------------------------------------------------------- 1. local pass
// grid (nwave, nchunk, nseq), 64 threads.  Chunk-local state H (zero start), decay sum S,
// chunk-local adjoint E (zero end).
namespace bwd {

// An element as stored (bf16 bits or float) and its float value.
template <class Io>
__device__ inline float widen(typename Io::T r)
{
    if constexpr (sizeof(typename Io::T) == 2)
        return __uint_as_float(static_cast<uint32_t>(r) << 16);
    else
        return r;
}

// v unchanged, but computed by here: an empty asm that reads and writes it.
__device__ inline void hold(float &v) { asm volatile("" : "+v"(v)); }

// The B_t or C_t row (as row16), its load issued only once dep (uniform) and vdep (per lane)
// are known: the empty asm ties the row's address to both.  Scalar loads of read-only rows
// are otherwise hoisted to the top of an unrolled chunk, more rows than there are scalar
// registers (spilled to vector lanes).
template <class Io, bool kFullN>
__device__ inline void row16_after(const void *p, size_t t, int N, float dep, float vdep, float *f)
{
    asm volatile("" : "+s"(p) : "s"(dep), "v"(vdep));
    row16<Io, kFullN>(p, t, N, f);
}

// Local pass over one chunk, one sweep in time order.  The zero-end adjoint needs no reverse
// sweep: unrolling E = Abar_0 (gy_0 C_0 + Abar_1 (gy_1 C_1 + ...)) gives
// E = sum_i P_i gy_i C_i with P_i = Abar_0 ... Abar_i, a running product of the factors the
// forward computes anyway (one multiply per state and token instead of a second exp).
// kFull (all kChunk tokens present): the chunk's x, dt, dout and z of this lane's channel
// are loaded in one batch before any arithmetic (one memory latency per chunk instead of one
// per token and input), and token i+1's B / C rows are loaded while token i is computed.  A
// partial chunk (the last of a sequence) loads token by token.
template <class Io, bool kFullN, bool kFull>
__device__ inline void local_chunk(const BwdArgs &a, int s, int c, int d, bool dok, int dc, size_t t0, int cs, int n_t)
{
    using T = typename Io::T;
    constexpr int kR = kFull ? kChunk : 1;  // batched registers (unused for a partial chunk)
    Chan ch;
    load_chan(a, dc, ch);
    const bool has_z = a.z != nullptr;

    float xm3 = x_at<Io>(a, s, t0, cs - 3, dc), xm2 = x_at<Io>(a, s, t0, cs - 2, dc), xm1 = x_at<Io>(a, s, t0, cs - 1, dc);
    T xr[kR], dr[kR], gr[kR], zr[kR];
    float bn[kMaxState], cn[kMaxState];  // B / C rows of the next token (kFull)
    if constexpr (kFull) {
        const size_t base = (t0 + static_cast<size_t>(cs)) * a.D + dc;
        const T *px = static_cast<const T *>(a.x), *pd = static_cast<const T *>(a.dt);
        const T *pg = static_cast<const T *>(a.dout);
        const T *pz = has_z ? static_cast<const T *>(a.z) : pg;  // without a gate: loaded, unused
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            xr[i] = px[base + static_cast<size_t>(i) * a.D];
            dr[i] = pd[base + static_cast<size_t>(i) * a.D];
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            gr[i] = pg[base + static_cast<size_t>(i) * a.D];
            zr[i] = pz[base + static_cast<size_t>(i) * a.D];
        }
        row16<Io, kFullN>(a.B, t0 + cs, a.N, bn);
        row16<Io, kFullN>(a.C, t0 + cs, a.N, cn);
        __builtin_amdgcn_sched_barrier(0);
    }

    float h[kMaxState], P[kMaxState], E[kMaxState];
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) {
        h[n] = 0.0f;
        P[n] = 1.0f;
        E[n] = 0.0f;
    }
    float S = 0.0f;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        if (kFull || i < n_t) {
            const size_t t = t0 + static_cast<size_t>(cs + i);
            float xt, dtv, gy, b[kMaxState], cr[kMaxState];
            if constexpr (kFull) {
#pragma unroll
                for (int n = 0; n < kMaxState; ++n) {
                    b[n] = bn[n];
                    cr[n] = cn[n];
                }
                if (i + 1 < kChunk) {  // after this token's rows and the previous token's states
                    const float dep = b[kMaxState - 1] + cr[kMaxState - 1];
                    row16_after<Io, kFullN>(a.B, t + 1, a.N, dep, h[kMaxState - 1], bn);
                    row16_after<Io, kFullN>(a.C, t + 1, a.N, dep, h[kMaxState - 1], cn);
                }
                xt = widen<Io>(xr[i]);
                dtv = widen<Io>(dr[i]);
                const float g = widen<Io>(gr[i]);
                gy = has_z ? gate_grad(g, true, widen<Io>(zr[i])) : g;
            } else {
                xt = Io::ld(a.x, t * a.D + dc);
                dtv = Io::ld(a.dt, t * a.D + dc);
                const float g = Io::ld(a.dout, t * a.D + dc);
                gy = gate_grad(g, has_z, has_z ? Io::ld(a.z, t * a.D + dc) : 0.0f);
                row16<Io, kFullN>(a.B, t, a.N, b);
                row16<Io, kFullN>(a.C, t, a.N, cr);
            }
            Front f;
            front(ch, xm3, xm2, xm1, xt, dtv, f);
            xm3 = xm2;
            xm2 = xm1;
            xm1 = xt;
            const float du = (f.lg * kLn2) * f.u;
#pragma unroll
            for (int n = 0; n < kMaxState; ++n) {
                const float ab = hw_exp2(f.lg * ch.A[n]);
                h[n] = __builtin_fmaf(ab, h[n], du * b[n]);
                P[n] *= ab;
                E[n] = __builtin_fmaf(P[n], gy * cr[n], E[n]);
            }
            S += f.lg;
        }
        if constexpr (kFull) {
            // one token at a time: its states are computed here, not sunk towards the stores
            // at the end (which would keep every token's rows alive until then)
#pragma unroll
            for (int n = 0; n < kMaxState; ++n) {
                hold(h[n]);
                hold(P[n]);
                hold(E[n]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (dok) {
        const size_t o = ((static_cast<size_t>(s) * a.nchunk + c) * a.D + d);
        float4 *ph = reinterpret_cast<float4 *>(a.hck + o * kMaxState);
        float4 *pe = reinterpret_cast<float4 *>(a.eck + o * kMaxState);
#pragma unroll
        for (int g = 0; g < kMaxState / 4; ++g) {
            ph[g] = make_float4(h[4 * g], h[4 * g + 1], h[4 * g + 2], h[4 * g + 3]);
            pe[g] = make_float4(E[4 * g], E[4 * g + 1], E[4 * g + 2], E[4 * g + 3]);
        }
        a.lsum[o] = S;
    }
}

}  // namespace bwd

template <class Io, bool kFullN>
__global__ __launch_bounds__(bwd::kLanes) void bwd_local_kernel(BwdArgs a)
{
    using namespace bwd;
    const int s = blockIdx.z, c = blockIdx.y;
    const int d = blockIdx.x * kLanes + threadIdx.x;
    const bool dok = d < a.D;
    const int dc = dok ? d : a.D - 1;
    size_t t0, t1;
    seq_bounds(a, s, t0, t1);
    const int L = static_cast<int>(t1 - t0);
    const int cs = c * kChunk;
    if (cs >= L) return;  // chunk past this sequence's end (uniform)
    const int n_t = min(kChunk, L - cs);
    if (n_t == kChunk)  // uniform
        local_chunk<Io, kFullN, true>(a, s, c, d, dok, dc, t0, cs, n_t);
    else
        local_chunk<Io, kFullN, false>(a, s, c, d, dok, dc, t0, cs, n_t);
}

// ---------------------------------------------------------------- 2. carry pass
// grid (ceil(D * 16 / 256), nseq), 256 threads: one lane per (sequence, channel, state),
// sequential over chunks, the loads kPre chunks ahead (the loop body is one exp and one
// FMA, so it is load-latency bound).  hck becomes the state entering each chunk, eck the
// adjoint entering it from the right (stored for the last chunk of each full-pass group,
// the only ones read); the gradient of h0 is what is left at the start.
__global__ __launch_bounds__(256) void bwd_carry_kernel(BwdArgs a)
{
    using namespace bwd;
    constexpr int kPre = 4;
    const int s = blockIdx.y;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int d = idx >> 4, n = idx & (kMaxState - 1);
    if (d >= a.D) return;  // no barriers: an early exit is safe
    size_t t0, t1;
    seq_bounds(a, s, t0, t1);
    const int L = static_cast<int>(t1 - t0);
    const int nc = min((L + kChunk - 1) / kChunk, a.nchunk);  // clamped: offsets are caller data
    const bool on = n < a.N;
    const float An = on ? a.A[static_cast<size_t>(d) * a.N + n] : 0.0f;
    const size_t hb = (static_cast<size_t>(s) * a.D + d) * a.N + n;
    float h = (on && a.h0 != nullptr) ? a.h0[hb] : 0.0f;
    float R = (on && a.dh_final != nullptr) ? a.dh_final[hb] : 0.0f;
    const size_t base = static_cast<size_t>(s) * a.nchunk * a.D + d;  // chunk c: base + c * D
    auto at = [&](int c) { return base + static_cast<size_t>(c) * a.D; };
    // forward over chunks
    {
        float Hq[kPre], Sq[kPre];
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
            const int c = min(k, max(nc - 1, 0));
            Hq[k] = nc > 0 ? a.hck[at(c) * kMaxState + n] : 0.0f;
            Sq[k] = nc > 0 ? a.lsum[at(c)] : 0.0f;
        }
        for (int c0 = 0; c0 < nc; c0 += kPre) {
#pragma unroll
            for (int k = 0; k < kPre; ++k) {
                const int c = c0 + k;
                if (c < nc) {
                    const float H = Hq[k], S = Sq[k];
                    const int cn = min(c + kPre, nc - 1);  // refill (clamped re-load at the end)
                    Hq[k] = a.hck[at(cn) * kMaxState + n];
                    Sq[k] = a.lsum[at(cn)];
                    a.hck[at(c) * kMaxState + n] = h;
                    h = __builtin_fmaf(hw_exp2(An * S), h, H);
                }
            }
        }
    }
    // reverse over chunks
    {
        float Eq[kPre], Sq[kPre];
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
            const int c = max(nc - 1 - k, 0);
            Eq[k] = nc > 0 ? a.eck[at(c) * kMaxState + n] : 0.0f;
            Sq[k] = nc > 0 ? a.lsum[at(c)] : 0.0f;
        }
        for (int c0 = nc - 1; c0 >= 0; c0 -= kPre) {
#pragma unroll
            for (int k = 0; k < kPre; ++k) {
                const int c = c0 - k;
                if (c >= 0) {
                    const float E = Eq[k], S = Sq[k];
                    const int cn = max(c - kPre, 0);
                    Eq[k] = a.eck[at(cn) * kMaxState + n];
                    Sq[k] = a.lsum[at(cn)];
                    if (c % kGroup == kGroup - 1 || c == nc - 1) a.eck[at(c) * kMaxState + n] = R;  // read at group ends only
                    R = __builtin_fmaf(hw_exp2(An * S), R, E);
                }
            }
        }
    }
    if (a.dh0 != nullptr && on) a.dh0[hb] = R;
}

// ---------------------------------------------------------------- 3. full pass
// grid (nwave, ngroup, nseq), 64 threads: one wave, so the LDS reduction of dB / dC is the
// wave's own and needs no workgroup barrier (LDS operations of one wave take effect in
// order).  A lane takes a group of kGroup consecutive chunks, last to first, carrying the
// adjoint from one chunk into the previous one.  Within a chunk, sub-chunks of kSub tokens
// are handled last to first: the forward recomputed from the chunk's true start or from a
// checkpoint, then the reverse with every per-token gradient.  The first pass over a full
// chunk (sub-chunk kNSub-1) walks tokens 0 .. 15 and leaves the states after tokens 4 and 8
// in LDS, so sub-chunks 2 and 1 recompute only their own 4 tokens (28 forward tokens per
// chunk instead of 40); a partial chunk (the last of a sequence) recomputes every sub-chunk
// from the chunk start.
namespace bwd {

template <int V>
struct IntTag {
    static constexpr int value = V;
};

// One forward token: front end, then h <- Abar h + Delta u B; the x history shifts by one.
__device__ inline void fwd_step(const Chan &ch, float &xm3, float &xm2, float &xm1, float xt, float dtv,
                                const float *b, float *h, Front &f)
{
    front(ch, xm3, xm2, xm1, xt, dtv, f);
    xm3 = xm2;
    xm2 = xm1;
    xm1 = xt;
    const float du = (f.lg * kLn2) * f.u;
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) h[n] = __builtin_fmaf(hw_exp2(f.lg * ch.A[n]), h[n], du * b[n]);
}

// Per-lane accumulators of the reverse.
struct RevAcc {
    float R[kMaxState];  // adjoint of the state after the token being reversed
    float dA[kMaxState];
    float dD, dbias;
};

// Per-lane constants of the reverse.
struct RevCtx {
    float *tile;   // LDS [kLanes][kTilePitch]
    float *trow;   // this lane's row of it
    int ro, rp;    // reduction: column ro, half rp of the lanes
    int wv;        // channel wave
    bool dok;      // a real channel (not padding)
    bool has_z;
};

// Order of this wave's LDS accesses without waiting for them: LDS operations of one wave take
// effect in issue order, so the compiler only has to keep them in program order.
__device__ inline void wave_lds_order()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Reverse of one token t (ix = its element): dz, ddt, dpre stored; the adjoint carried to the
// token before; dA, dD, dbias accumulated; dB / dC summed over the wave's 64 channels through
// the LDS tile and stored as this wave's partial.  hcur / hprev: states after / before it.
template <class Io>
__device__ inline void rev_step(const BwdArgs &a, const Chan &ch, const RevCtx &rc, const Front &f, float g, float zv,
                                const float *br, const float *cr, const float *hcur, const float *hprev, size_t t,
                                size_t ix, RevAcc &ac)
{
    const float delta = f.lg * kLn2;
    // Abar recomputed from a copy of lg the compiler cannot see through: otherwise it keeps
    // the forward's exp2(lg A) of the sub-chunk's tokens alive until here (64 registers).
    float lgr = f.lg;
    hold(lgr);
    float y = ch.dsk * f.u;
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) y = __builtin_fmaf(cr[n], hcur[n], y);
    float gy = g;
    if (rc.has_z) {
        const float sz = sigmoid(zv);
        const float dzv = g * y * sz * __builtin_fmaf(zv, 1.0f - sz, 1.0f);
        if (rc.dok) Io::st(a.dz, ix, dzv);
        gy = g * (zv * sz);
    }
    ac.dD = __builtin_fmaf(gy, f.u, ac.dD);
    float S1 = 0.0f, S2 = 0.0f;
    const float dun = rc.dok ? delta * f.u : 0.0f;  // padding channels add zeros to dB / dC
    const float gyc = rc.dok ? gy : 0.0f;
    wave_lds_order();  // the previous token's tile reads come first
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) {
        const float abar = hw_exp2(lgr * ch.A[n]);
        const float G = __builtin_fmaf(gy, cr[n], ac.R[n]);
        const float ga = G * abar;
        const float q = ga * hprev[n];
        S1 = __builtin_fmaf(q, ch.A[n], S1);
        ac.dA[n] = __builtin_fmaf(q, delta, ac.dA[n]);
        S2 = __builtin_fmaf(G, br[n], S2);
        ac.R[n] = ga;
        rc.trow[n] = G * dun;
        rc.trow[kMaxState + n] = gyc * hcur[n];
    }
    const float ddel = __builtin_fmaf(f.u, S2, S1);
    const float du = __builtin_fmaf(delta, S2, gy * ch.dsk);
    const float da = ddel * sigmoid(f.a);
    ac.dbias += da;
    const float sp = sigmoid(f.pre);
    const float dpre = du * sp * __builtin_fmaf(f.pre, 1.0f - sp, 1.0f);
    if (rc.dok) {
        Io::st(a.ddt, ix, da);
        a.dpre[ix] = dpre;
    }
    // dB / dC: column ro over half rp of the lanes (the 32 reads issued together), then the
    // halves added across lanes l and l ^ 32
    wave_lds_order();
    float v[32];
#pragma unroll
    for (int l = 0; l < 32; ++l) v[l] = rc.tile[(rc.rp * 32 + l) * kTilePitch + rc.ro];
    float acc = 0.0f;
#pragma unroll
    for (int l = 0; l < 32; ++l) acc += v[l];
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
    acc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    __attribute__((address_space(1))) float *pb = (__attribute__((address_space(1))) float *)a.pbc;
    asm volatile("" : "+s"(pb));  // the lane's address recomputed, not kept (or spilled) from earlier tokens
    if (rc.rp == 0) pb[(t * a.nwave + rc.wv) * kBC + rc.ro] = acc;
}

__device__ inline void hold_all(float *v)
{
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) hold(v[n]);
}

// A full chunk (all kChunk tokens).  Each sub-chunk's x, dt, dout and z come in one batch of
// loads: the first sub-chunk's issued at the chunk start, every later one's during the two
// last reverse tokens of the sub-chunk before it (the states of its two first tokens are dead
// by then, which leaves the registers), so its memory latency overlaps arithmetic.  B / C rows
// are loaded one token ahead; every token ends with its states held and a scheduling
// barrier, so the compiler neither hoists later rows (scalar registers) nor sinks earlier
// arithmetic.
template <class Io, bool kFullN>
__device__ inline void full_chunk16(const BwdArgs &a, const Chan &ch, const RevCtx &rc, int s, size_t t0, int c,
                                   int dc, int lane, float (*ck)[kMaxState][kLanes], RevAcc &ac)
{
    using T = typename Io::T;
    const int cs = c * kChunk;
    const size_t base = (t0 + static_cast<size_t>(cs)) * a.D + dc;  // token 0 of the chunk, this channel
    const float4 *phc = reinterpret_cast<const float4 *>(a.hck + ((static_cast<size_t>(s) * a.nchunk + c) * a.D + dc) * kMaxState);
    const T *px = static_cast<const T *>(a.x), *pd = static_cast<const T *>(a.dt);
    const T *pg = static_cast<const T *>(a.dout);
    const T *pz = rc.has_z ? static_cast<const T *>(a.z) : pg;  // without a gate: loaded, unused
    const float xc3 = x_at<Io>(a, s, t0, cs - 3, dc), xc2 = x_at<Io>(a, s, t0, cs - 2, dc);
    const float xc1 = x_at<Io>(a, s, t0, cs - 1, dc);
    const size_t tc = t0 + static_cast<size_t>(cs);  // token 0 of the chunk

    // The inputs of one sub-chunk J (tokens w0 .. e0 + kSub - 1 of x and dt, the x history
    // before w0 when w0 > 0, dout and z of its own tokens; h: the chunk's start state, for
    // the sub-chunks that start there).
    struct Batch {
        T xr[kChunk], dr[kChunk], hx[3], gr[kSub], zr[kSub];
        float h[kMaxState];
    };
    auto load_in = [&](auto jtag, Batch &b) __attribute__((always_inline)) {
        constexpr int J = decltype(jtag)::value;
        constexpr int e0 = J * kSub;
        constexpr int w0 = (J == 1 || J == 2) ? e0 : 0;
        constexpr int nx = e0 + kSub - w0;
        // the bases pass through an empty asm per batch, so the compiler recomputes the
        // addresses instead of keeping earlier batches' alive (two registers each)
        using GPtr = const __attribute__((address_space(1))) T *;  // global: not flat (flat loads count as LDS too)
        GPtr qx = (GPtr)px, qd = (GPtr)pd, qg = (GPtr)pg, qz = (GPtr)pz;
        asm volatile("" : "+s"(qx), "+s"(qd), "+s"(qg), "+s"(qz));
#pragma unroll
        for (int k = 0; k < nx; ++k) {
            b.xr[k] = qx[base + static_cast<size_t>(w0 + k) * a.D];
            b.dr[k] = qd[base + static_cast<size_t>(w0 + k) * a.D];
        }
        if constexpr (w0 > 0) {
#pragma unroll
            for (int k = 0; k < 3; ++k) b.hx[k] = qx[base + static_cast<size_t>(w0 - 3 + k) * a.D];
        }
#pragma unroll
        for (int e = 0; e < kSub; ++e) {
            b.gr[e] = qg[base + static_cast<size_t>(e0 + e) * a.D];
            b.zr[e] = qz[base + static_cast<size_t>(e0 + e) * a.D];
        }
    };
    auto load_h = [&](Batch &b) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < kMaxState / 4; ++g) {
            const float4 q = phc[g];
            b.h[4 * g] = q.x;
            b.h[4 * g + 1] = q.y;
            b.h[4 * g + 2] = q.z;
            b.h[4 * g + 3] = q.w;
        }
    };

    // Sub-chunk J from its batch b; issues the next sub-chunk's batch into nb.
    auto sub = [&](auto jtag, Batch &b, Batch &nb) __attribute__((always_inline)) {
        constexpr int J = decltype(jtag)::value;
        constexpr int e0 = J * kSub;                          // first own token
        constexpr int w0 = (J == 1 || J == 2) ? e0 : 0;       // first token recomputed
        constexpr bool from_hc = J == 0 || J == kNSub - 1;    // else from checkpoint J - 1
        float bn[kMaxState], cn[kMaxState];
        row16_after<Io, kFullN>(a.B, tc + w0, a.N, 0.0f, ac.R[kMaxState - 1], bn);
        __builtin_amdgcn_sched_barrier(0);
        float h[kMaxState];
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) h[n] = from_hc ? b.h[n] : ck[J > 0 ? J - 1 : 0][n][lane];
        float xm3 = xc3, xm2 = xc2, xm1 = xc1;
        if constexpr (w0 > 0) {
            xm3 = widen<Io>(b.hx[0]);
            xm2 = widen<Io>(b.hx[1]);
            xm1 = widen<Io>(b.hx[2]);
        }
        // ---- earlier sub-chunks: states only (the first pass keeps two checkpoints)
#pragma unroll
        for (int i = w0; i < e0; ++i) {
            float bb[kMaxState];
#pragma unroll
            for (int n = 0; n < kMaxState; ++n) bb[n] = bn[n];
            row16_after<Io, kFullN>(a.B, tc + i + 1, a.N, bb[kMaxState - 1], h[kMaxState - 1], bn);
            Front f;
            fwd_step(ch, xm3, xm2, xm1, widen<Io>(b.xr[i - w0]), widen<Io>(b.dr[i - w0]), bb, h, f);
            if constexpr (J == kNSub - 1) {
                if ((i + 1) % kSub == 0 && (i + 1) / kSub < kNSub - 1) {
#pragma unroll
                    for (int n = 0; n < kMaxState; ++n) ck[(i + 1) / kSub - 1][n][lane] = h[n];
                }
            }
            hold_all(h);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- own tokens forward
        float hp[kMaxState], hs[kSub][kMaxState];
        Front fs[kSub];
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) hp[n] = h[n];
#pragma unroll
        for (int e = 0; e < kSub; ++e) {
            float bb[kMaxState];
#pragma unroll
            for (int n = 0; n < kMaxState; ++n) bb[n] = bn[n];
            if (e + 1 < kSub) {
                row16_after<Io, kFullN>(a.B, tc + e0 + e + 1, a.N, bb[kMaxState - 1], h[kMaxState - 1], bn);
            } else {  // the reverse starts with this token: keep its B row, load its C row
                row16_after<Io, kFullN>(a.C, tc + e0 + e, a.N, bb[kMaxState - 1], h[kMaxState - 1], cn);
            }
            const int i = e0 + e - w0;
            fwd_step(ch, xm3, xm2, xm1, widen<Io>(b.xr[i]), widen<Io>(b.dr[i]), bb, h, fs[e]);
#pragma unroll
            for (int n = 0; n < kMaxState; ++n) hs[e][n] = h[n];
            hold_all(h);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- reverse
#pragma unroll
        for (int e = kSub - 1; e >= 0; --e) {
            if constexpr (J > 0) {  // the next sub-chunk's batch
                if (e == 1) load_in(IntTag<J - 1>{}, nb);
                if (J == 1 && e == 0) load_h(nb);
            }
            float br[kMaxState], cr[kMaxState];
#pragma unroll
            for (int n = 0; n < kMaxState; ++n) {
                br[n] = bn[n];
                cr[n] = cn[n];
            }
            if (e > 0) {
                const float dep = br[kMaxState - 1] + cr[kMaxState - 1];
                row16_after<Io, kFullN>(a.B, tc + e0 + e - 1, a.N, dep, ac.R[kMaxState - 1], bn);
                row16_after<Io, kFullN>(a.C, tc + e0 + e - 1, a.N, dep, ac.R[kMaxState - 1], cn);
            }
            const size_t t = tc + static_cast<size_t>(e0 + e);
            rev_step<Io>(a, ch, rc, fs[e], widen<Io>(b.gr[e]), widen<Io>(b.zr[e]), br, cr, hs[e], e > 0 ? hs[e > 0 ? e - 1 : 0] : hp,
                         t, base + static_cast<size_t>(e0 + e) * a.D, ac);
            hold_all(ac.R);
            hold_all(ac.dA);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    Batch b3, b2, b1, b0;
    load_in(IntTag<3>{}, b3);
    load_h(b3);
    sub(IntTag<3>{}, b3, b2);
    sub(IntTag<2>{}, b2, b1);
    sub(IntTag<1>{}, b1, b0);
    sub(IntTag<0>{}, b0, b3);  // (issues nothing)
}

// A partial chunk (n_t < kChunk tokens, the last of a sequence): every sub-chunk recomputes
// the forward from the chunk start, token by token.
template <class Io, bool kFullN>
__device__ inline void part_chunk(const BwdArgs &a, const Chan &ch, const RevCtx &rc, int s, size_t t0, int c, int n_t,
                                  int dc, RevAcc &ac)
{
    const int cs = c * kChunk;
    float hc[kMaxState];
    {
        const float4 *ph = reinterpret_cast<const float4 *>(a.hck + ((static_cast<size_t>(s) * a.nchunk + c) * a.D + dc) * kMaxState);
#pragma unroll
        for (int g = 0; g < kMaxState / 4; ++g) {
            const float4 q = ph[g];
            hc[4 * g] = q.x;
            hc[4 * g + 1] = q.y;
            hc[4 * g + 2] = q.z;
            hc[4 * g + 3] = q.w;
        }
    }
    const float xc3 = x_at<Io>(a, s, t0, cs - 3, dc), xc2 = x_at<Io>(a, s, t0, cs - 2, dc);
    const float xc1 = x_at<Io>(a, s, t0, cs - 1, dc);
#pragma unroll
    for (int j = kNSub - 1; j >= 0; --j) {
        if (j * kSub >= n_t) continue;  // uniform
        float h[kMaxState], hp[kMaxState], hs[kSub][kMaxState];
        Front fs[kSub];
        float xm3 = xc3, xm2 = xc2, xm1 = xc1;
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) h[n] = hc[n];
        for (int i = 0; i < j * kSub; ++i) {  // earlier sub-chunks: states only
            const size_t t = t0 + static_cast<size_t>(cs + i);
            float b[kMaxState];
            row16<Io, kFullN>(a.B, t, a.N, b);
            Front f;
            fwd_step(ch, xm3, xm2, xm1, Io::ld(a.x, t * a.D + dc), Io::ld(a.dt, t * a.D + dc), b, h, f);
        }
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) hp[n] = h[n];
#pragma unroll
        for (int e = 0; e < kSub; ++e) {
            const int i = j * kSub + e;
            fs[e] = Front{0.0f, 0.0f, 0.0f, 0.0f};
            if (i < n_t) {
                const size_t t = t0 + static_cast<size_t>(cs + i);
                float b[kMaxState];
                row16<Io, kFullN>(a.B, t, a.N, b);
                fwd_step(ch, xm3, xm2, xm1, Io::ld(a.x, t * a.D + dc), Io::ld(a.dt, t * a.D + dc), b, h, fs[e]);
            }
#pragma unroll
            for (int n = 0; n < kMaxState; ++n) hs[e][n] = h[n];
        }
#pragma unroll
        for (int e = kSub - 1; e >= 0; --e) {
            const int i = j * kSub + e;
            if (i >= n_t) continue;  // uniform
            const size_t t = t0 + static_cast<size_t>(cs + i);
            const size_t ix = t * a.D + dc;
            float br[kMaxState], cr[kMaxState];
            row16<Io, kFullN>(a.B, t, a.N, br);
            row16<Io, kFullN>(a.C, t, a.N, cr);
            const float g = Io::ld(a.dout, ix);
            const float zv = rc.has_z ? Io::ld(a.z, ix) : 0.0f;
            rev_step<Io>(a, ch, rc, fs[e], g, zv, br, cr, hs[e], e > 0 ? hs[e > 0 ? e - 1 : 0] : hp, t, ix, ac);
        }
    }
}

}  // namespace bwd

template <class Io, bool kFullN>
__global__ __launch_bounds__(bwd::kLanes, 2) void bwd_full_kernel(BwdArgs a)
{
    using namespace bwd;
    __shared__ float tile[kLanes * kTilePitch];
    // States after 4 and 8 tokens of a full chunk (lane-private, lane fastest).
    __shared__ float ck[kNSub - 2][kMaxState][kLanes];
    const int s = blockIdx.z, cg = blockIdx.y, wv = blockIdx.x;
    const int lane = threadIdx.x;
    const int d = wv * kLanes + lane;
    const bool dok = d < a.D;
    const int dc = dok ? d : a.D - 1;
    size_t t0, t1;
    seq_bounds(a, s, t0, t1);
    const int L = static_cast<int>(t1 - t0);
    const int nc = min((L + kChunk - 1) / kChunk, a.nchunk);
    const int cfirst = cg * kGroup;
    if (cfirst >= nc) {  // uniform over the workgroup (one wave): an empty slot adds zeros
        if (dok) {
            float *pp = a.ppar + ((static_cast<size_t>(s) * a.ngroup + cg) * a.D + d) * kPar;
#pragma unroll
            for (int k = 0; k < kPar; ++k) pp[k] = 0.0f;
        }
        return;
    }
    const int clast = min(cfirst + kGroup, nc) - 1;
    Chan ch;
    load_chan(a, dc, ch);
    const RevCtx rc{tile, tile + lane * kTilePitch, lane & 31, lane >> 5, wv, dok, a.z != nullptr};
    RevAcc ac;
    {
        const size_t o = (static_cast<size_t>(s) * a.nchunk + clast) * a.D + dc;
        const float4 *pe = reinterpret_cast<const float4 *>(a.eck + o * kMaxState);
#pragma unroll
        for (int g = 0; g < kMaxState / 4; ++g) {
            const float4 v = pe[g];
            ac.R[4 * g] = v.x;
            ac.R[4 * g + 1] = v.y;
            ac.R[4 * g + 2] = v.z;
            ac.R[4 * g + 3] = v.w;
        }
    }
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) ac.dA[n] = 0.0f;
    ac.dD = 0.0f;
    ac.dbias = 0.0f;
    for (int c = clast; c >= cfirst; --c) {
        const int n_t = min(kChunk, L - c * kChunk);
        if (n_t == kChunk)  // uniform
            full_chunk16<Io, kFullN>(a, ch, rc, s, t0, c, dc, lane, ck, ac);
        else
            part_chunk<Io, kFullN>(a, ch, rc, s, t0, c, n_t, dc, ac);
    }
    if (dok) {
        float *pp = a.ppar + ((static_cast<size_t>(s) * a.ngroup + cg) * a.D + d) * kPar;
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) pp[n] = ac.dA[n];
        pp[kMaxState] = ac.dD;
        pp[kMaxState + 1] = ac.dbias;
    }
}

// ---------------------------------------------------------------- 4. conv pass
// grid (nrun * nseq, ceil(D / 256)), 256 threads: one thread per (sequence, run of kRun
// tokens, channel).  dx_t = sum_k w_k dpre_{t+3-k} (+ dconv_final for the last three
// tokens), dconv0 for the inputs before the sequence, dconv_w / dconv_b partials.
template <class Io>
__global__ __launch_bounds__(256) void bwd_conv_kernel(BwdArgs a)
{
    using namespace bwd;
    const int s = blockIdx.x / a.nrun, r = blockIdx.x - s * a.nrun;
    const int d = blockIdx.y * 256 + threadIdx.x;
    if (d >= a.D) return;  // no barriers
    size_t t0, t1;
    seq_bounds(a, s, t0, t1);
    const int L = static_cast<int>(t1 - t0);
    const int tb = r * kRun;
    float *pc = a.pconv + ((static_cast<size_t>(s) * a.nrun + r) * a.D + d) * kConvPar;
    if (tb >= L && r > 0) {  // run 0 always runs (dconv0 of an empty sequence); empty runs add zeros
#pragma unroll
        for (int k = 0; k < kConvPar; ++k) pc[k] = 0.0f;
        return;
    }
    const int te = min(tb + kRun, L);
    const float4 w = *reinterpret_cast<const float4 *>(a.conv_w + static_cast<size_t>(d) * kConvK);
    auto dpre_at = [&](int tp) { return tp < L ? a.dpre[(t0 + static_cast<size_t>(tp)) * a.D + d] : 0.0f; };
    auto dcf_at = [&](int tt) {  // gradient of the outgoing history entry holding token tt
        return (a.dconv_final != nullptr && tt >= L - 3 && tt < L)
                   ? Io::ld(a.dconv_final, (static_cast<size_t>(s) * 3 + static_cast<size_t>(tt - (L - 3))) * a.D + d)
                   : 0.0f;
    };
    // windows: dp[k] = dpre of token t+k, xw[k] = x of token t-3+k
    float dp0 = dpre_at(tb), dp1 = dpre_at(tb + 1), dp2 = dpre_at(tb + 2), dp3 = dpre_at(tb + 3);
    float xw0 = x_at<Io>(a, s, t0, tb - 3, d), xw1 = x_at<Io>(a, s, t0, tb - 2, d), xw2 = x_at<Io>(a, s, t0, tb - 1, d);
    float pw0 = 0.0f, pw1 = 0.0f, pw2 = 0.0f, pw3 = 0.0f, pb = 0.0f;
    for (int t = tb; t < te; ++t) {
        const size_t ix = (t0 + static_cast<size_t>(t)) * a.D + d;
        const float xt = Io::ld(a.x, ix);
        float g = __builtin_fmaf(w.w, dp0, __builtin_fmaf(w.z, dp1, __builtin_fmaf(w.y, dp2, w.x * dp3)));
        if (t >= L - 3) g += dcf_at(t);  // uniform over the workgroup
        Io::st(a.dx, ix, g);
        pb += dp0;
        pw0 = __builtin_fmaf(dp0, xw0, pw0);
        pw1 = __builtin_fmaf(dp0, xw1, pw1);
        pw2 = __builtin_fmaf(dp0, xw2, pw2);
        pw3 = __builtin_fmaf(dp0, xt, pw3);
        xw0 = xw1;
        xw1 = xw2;
        xw2 = xt;
        dp0 = dp1;
        dp1 = dp2;
        dp2 = dp3;
        dp3 = dpre_at(t + 4);
    }
    if (r == 0 && a.dconv0 != nullptr) {
        // history entry jj holds token jj - 3, whose input feeds the pre-activations of
        // tokens jj - 3 + 3 - k = jj - k through tap k
#pragma unroll
        for (int jj = 0; jj < 3; ++jj) {
            const float wk[kConvK] = {w.x, w.y, w.z, w.w};
            float g = dcf_at(jj - 3);
#pragma unroll
            for (int k = 0; k < kConvK; ++k)
                if (jj - k >= 0) g = __builtin_fmaf(wk[k], dpre_at(jj - k), g);
            Io::st(a.dconv0, (static_cast<size_t>(s) * 3 + jj) * a.D + d, g);
        }
    }
    pc[0] = pw0;
    pc[1] = pw1;
    pc[2] = pw2;
    pc[3] = pw3;
    pc[kConvK] = pb;
}

// ---------------------------------------------------------------- 5. reductions
// dB / dC: grid ceil(total * 32 / 256), one thread per (token, output).
template <class Io>
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(BwdArgs a)
{
    using namespace bwd;
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= static_cast<size_t>(a.total) * kBC) return;
    const size_t t = i / kBC;
    const int k = static_cast<int>(i - t * kBC);
    const int n = k & (kMaxState - 1);
    if (n >= a.N) return;
    float acc = 0.0f;
#pragma unroll 16
    for (int wv = 0; wv < a.nwave; ++wv) acc += a.pbc[(t * a.nwave + wv) * kBC + k];  // in wave order
    Io::st(k < kMaxState ? a.dB : a.dC, t * a.N + n, acc);
}

// Parameters, stage 1: column sums of a [rows][cols] partial matrix over the rows r = split
// (mod nsplit); grid (ceil(cols / 256), nsplit).  Stage 2 adds the nsplit sums in order, so
// the result does not depend on timing.
__global__ __launch_bounds__(256) void bwd_colsum_kernel(const float *__restrict__ m, int rows, int cols, int nsplit,
                                                        float *__restrict__ out)
{
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= cols) return;
    float acc = 0.0f;
    for (int r = blockIdx.y; r < rows; r += nsplit) acc += m[static_cast<size_t>(r) * cols + col];
    out[static_cast<size_t>(blockIdx.y) * cols + col] = acc;
}

// Parameters, stage 2: one thread per (channel, parameter), the nsplit sums added in order.
__global__ __launch_bounds__(256) void bwd_reduce_par_kernel(BwdArgs a)
{
    using namespace bwd;
    constexpr int kAll = kPar + kConvPar;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= a.D * kAll) return;
    const int d = i / kAll, k = i - d * kAll;
    float acc = 0.0f;
    if (k < kPar) {
#pragma unroll 8
        for (int sp = 0; sp < kSplit; ++sp) acc += a.par2[(static_cast<size_t>(sp) * a.D + d) * kPar + k];
        if (k < kMaxState) {
            if (k < a.N) a.dA[static_cast<size_t>(d) * a.N + k] = acc;
        } else if (k == kMaxState) {
            a.dD[d] = acc;
        } else {
            a.ddt_bias[d] = acc;
        }
    } else {
        const int kc = k - kPar;
#pragma unroll 8
        for (int sp = 0; sp < kSplit; ++sp) acc += a.conv2[(static_cast<size_t>(sp) * a.D + d) * kConvPar + kc];
        if (kc < kConvK)
            a.dconv_w[static_cast<size_t>(d) * kConvK + kc] = acc;
        else
            a.dconv_b[d] = acc;
    }
}

// ---------------------------------------------------------------- host side
// Workspace layout (offsets in floats), every part 256-byte aligned.
struct BwdWorkspace {
    size_t hck, eck, lsum, dpre, ppar, pbc, pconv, par2, conv2, total_bytes;
};

inline BwdWorkspace bwd_workspace(int nseq, int seqlen, int total, int D)
{
    using namespace bwd;
    auto al = [](size_t f) { return (f + 63) / 64 * 64; };
    const size_t nchunk = (static_cast<size_t>(seqlen) + kChunk - 1) / kChunk;
    const size_t ngroup = (nchunk + kGroup - 1) / kGroup;
    const size_t nrun = std::max<size_t>(1, (static_cast<size_t>(seqlen) + kRun - 1) / kRun);
    const size_t nwave = (static_cast<size_t>(D) + kLanes - 1) / kLanes;
    const size_t sc = static_cast<size_t>(nseq) * nchunk * D;
    BwdWorkspace w;
    size_t off = 0;
    w.hck = off;
    off += al(sc * kMaxState);
    w.eck = off;
    off += al(sc * kMaxState);
    w.lsum = off;
    off += al(sc);
    w.dpre = off;
    off += al(static_cast<size_t>(total) * D);
    w.ppar = off;
    off += al(static_cast<size_t>(nseq) * ngroup * D * kPar);
    w.pbc = off;
    off += al(static_cast<size_t>(total) * nwave * kBC);
    w.pconv = off;
    off += al(static_cast<size_t>(nseq) * nrun * D * kConvPar);
    w.par2 = off;
    off += al(static_cast<size_t>(kSplit) * D * kPar);
    w.conv2 = off;
    off += al(static_cast<size_t>(kSplit) * D * kConvPar);
    w.total_bytes = off * sizeof(float);
    return w;
}

inline void launch_backward(BwdArgs a, float *ws, samba_dtype io, hipStream_t stream)
{
    using namespace bwd;
    const BwdWorkspace w = bwd_workspace(a.nseq, a.seqlen, a.total, a.D);
    a.nchunk = (a.seqlen + kChunk - 1) / kChunk;
    a.nrun = std::max(1, (a.seqlen + kRun - 1) / kRun);
    a.nwave = (a.D + kLanes - 1) / kLanes;
    a.hck = ws + w.hck;
    a.eck = ws + w.eck;
    a.lsum = ws + w.lsum;
    a.dpre = ws + w.dpre;
    a.ppar = ws + w.ppar;
    a.pbc = ws + w.pbc;
    a.pconv = ws + w.pconv;
    a.par2 = ws + w.par2;
    a.conv2 = ws + w.conv2;
    a.ngroup = (a.nchunk + kGroup - 1) / kGroup;
    const bool full = a.N == kMaxState;
    const dim3 g3(a.nwave, std::max(1, a.nchunk), a.nseq), b64(kLanes);
    if (a.nchunk > 0) {
        if (io == SAMBA_BF16) {
            if (full) bwd_local_kernel<IoBf16, true><<<g3, b64, 0, stream>>>(a);
            else bwd_local_kernel<IoBf16, false><<<g3, b64, 0, stream>>>(a);
        } else {
            if (full) bwd_local_kernel<IoF32, true><<<g3, b64, 0, stream>>>(a);
            else bwd_local_kernel<IoF32, false><<<g3, b64, 0, stream>>>(a);
        }
    }
    bwd_carry_kernel<<<dim3((a.D * kMaxState + 255) / 256, a.nseq), 256, 0, stream>>>(a);
    if (a.nchunk > 0) {
        const dim3 gg(a.nwave, a.ngroup, a.nseq);
        if (io == SAMBA_BF16) {
            if (full) bwd_full_kernel<IoBf16, true><<<gg, b64, 0, stream>>>(a);
            else bwd_full_kernel<IoBf16, false><<<gg, b64, 0, stream>>>(a);
        } else {
            if (full) bwd_full_kernel<IoF32, true><<<gg, b64, 0, stream>>>(a);
            else bwd_full_kernel<IoF32, false><<<gg, b64, 0, stream>>>(a);
        }
    }
    const dim3 gc(static_cast<unsigned>(a.nrun) * static_cast<unsigned>(a.nseq), (a.D + 255) / 256);
    if (io == SAMBA_BF16) bwd_conv_kernel<IoBf16><<<gc, 256, 0, stream>>>(a);
    else bwd_conv_kernel<IoF32><<<gc, 256, 0, stream>>>(a);
    if (a.total > 0) {
        const size_t nbc = static_cast<size_t>(a.total) * kBC;
        const unsigned gb = static_cast<unsigned>((nbc + 255) / 256);
        if (io == SAMBA_BF16) bwd_reduce_bc_kernel<IoBf16><<<gb, 256, 0, stream>>>(a);
        else bwd_reduce_bc_kernel<IoF32><<<gb, 256, 0, stream>>>(a);
    }
    {
        const int pcols = a.D * kPar, ccols = a.D * kConvPar;
        if (a.nchunk > 0)
            bwd_colsum_kernel<<<dim3((pcols + 255) / 256, kSplit), 256, 0, stream>>>(a.ppar, a.nseq * a.ngroup, pcols,
                                                                                     kSplit, a.par2);
        else  // no chunk at all: the stage-2 sums read zeros
            bwd_colsum_kernel<<<dim3((pcols + 255) / 256, kSplit), 256, 0, stream>>>(a.ppar, 0, pcols, kSplit, a.par2);
        bwd_colsum_kernel<<<dim3((ccols + 255) / 256, kSplit), 256, 0, stream>>>(a.pconv, a.nseq * a.nrun, ccols,
                                                                                 kSplit, a.conv2);
    }
    bwd_reduce_par_kernel<<<(a.D * (kPar + kConvPar) + 255) / 256, 256, 0, stream>>>(a);
}

}  // namespace samba
