// scan_rows.h -- prefill with one 16-lane DPP row per channel (one lane per state):
// the pieces shared by the row kernels and the single-role row kernel.
//
// The recurrence of page 1 section 3.4 ("The State Space Model Update (S6)") is
// independent across channels and, within a channel, across the d_state = 16 state
// components; only the readout y_t = sum_n C_t[n] h_t[n] couples the states.  The row
// kernels therefore give every channel a row of 16 lanes (lane n owns state n) and walk
// the sequence in time, so a batch-1 prompt of d_inner = 4096 channels still yields
// 65536 lanes with no cross-workgroup carry and no recomputation.
//
// In the single-role kernel below every wave does all the work of its 4 channels; it is
// the row kernel for grids of more than one workgroup per CU, where two workgroups share
// each CU (scan_split.h holds the two-role kernel for smaller grids).  Work is organised
// in blocks of 16 tokens (one per lane of a row) and stages of kStage tokens:
//  * per stage, the workgroup stages B and C (shared by its 16 channels) into LDS as
//    float32 (B transposed to [state][token], C as token rows) and the x / dt / z rows
//    of its 16 channels (16-byte buffer loads bounded by the stage's extent), with the
//    loads of the next stage issued at the start of the current one;
//  * per block, lane j runs the per-token front end for token t0+j: causal conv with the
//    taps x_{t-1..t-3} fetched from neighbouring lanes by DPP row rotations, SiLU,
//    softplus(dt + b); then all 16 lanes step their state through the 16 tokens,
//    receiving Delta and Delta*u of token t from lane t by DPP row broadcast fused into
//    the multiply;
//  * the 16x16 tile of states h_t[n] is transposed through LDS so that lane j sums the
//    readout of token t0+j against its C row, adds D*u, applies the SiLU(z) gate and
//    stores the output.
// The LDS traffic is software-pipelined: the B columns of block k+1 are read while block
// k computes, and the states of block k-1 are read before block k's recurrence and
// consumed after it.
#pragma once

#include "scan_common.h"

namespace samba {

namespace rows {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kRowsPerWave = 4;           // channels per wave (4 rows of 16 lanes)
constexpr int kChannels = kWaves * kRowsPerWave;  // channels per workgroup
constexpr int kBlock = 16;                // tokens per block (one per lane of a row)
// Single-role kernel's state tiles and C rows: one token's 16 values are a 64-byte row whose 16-byte chunk q sits
// at chunk q ^ tswz(t); a channel's 16 x 16 tile is followed by 16 floats of padding.
// Measured with rocprofv3 on gfx950 (probe kernels of these exact access patterns): the
// token lanes' 16-byte reads of 16 rows spent half their LDS cycles in bank conflicts with
// the earlier 80-byte padded rows and none with this layout, and the state lanes' 4-byte
// writes (one token, 16 states x 4 channels per wave) stay conflict-free.
constexpr int kPPitch = kBlock;
constexpr int kRowPitch = kBlock * kPPitch + 16;
__device__ constexpr int tswz(int t) { return (t >> 2) & 3; }
// float offset, within a token row, of value n (chunk n / 4 swizzled by the token's tswz = k)
__device__ inline int row_elem(int n, int k) { return (((n >> 2) ^ k) << 2) + (n & 3); }
constexpr int kStagerThreads = 256;       // threads that move one stage (B/C or token words)

// Logical workgroup index (sequence-major, then 16-channel block) of hardware workgroup h.
// Consecutive hardware ids go round-robin to the 8 XCDs, each with its own L2.  Groups of
// 4 consecutive logical blocks (64 channels: the 128-byte bf16 rows of x, dt, z and y they
// share) are placed on one XCD, and logical order otherwise follows dispatch order, so that
// a grid of several sequences is spread evenly over the XCDs.
__device__ inline int logical_block(int h, int nb)
{
    if (h >= (nb & ~31)) return h;
    const int i = h >> 5, x = h & 7, k = (h >> 3) & 3;
    return (i << 5) | (x << 2) | k;
}

// DPP controls (gfx9 encoding).
constexpr int kRowRor = 0x120;      // row_ror:k = kRowRor + k  (k = 1..15)
constexpr int kRowNewBcast = 0x150; // row_newbcast:k = kRowNewBcast + k

// DPP move with every source lane valid (row rotations and row broadcasts), so the
// compiler may fold it into the consuming VOP2 instruction.
template <int kCtrl>
__device__ inline float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, true));
}

// x_{t-s} for the lane's token: from lane j-s of this block, or lane 16+j-s of the previous
// block when j < s (row rotation of a per-lane select).
template <int kS>
__device__ inline float tap(float xcur, float xprev, int j)
{
    const float r = (j <= 15 - kS) ? xcur : xprev;
    return dpp<kRowRor + kS>(r);
}

// Compiler-level ordering point for the intra-wave LDS exchange (a wave executes its LDS
// instructions in order, so nothing is needed in hardware).
__device__ inline void wave_order()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Values loaded from LDS one step ahead pass through an empty asm statement after the
// step's barrier: the compiler then cannot start the next step's arithmetic on them inside
// the current step, right after the loads, where it would wait for their latency.
__device__ inline void hold(float &v) { asm volatile("" : "+v"(v)); }
__device__ inline void hold(uint16_t &v) { asm volatile("" : "+v"(v)); }
__device__ inline void hold(uint32_t &v) { asm volatile("" : "+v"(v)); }
__device__ inline void hold(uint4 &v)
{
    hold(v.x);
    hold(v.y);
    hold(v.z);
    hold(v.w);
}
__device__ inline void hold(float4 &v)
{
    hold(v.x);
    hold(v.y);
    hold(v.z);
    hold(v.w);
}

// Token tiles hold, per stage, x / dt / z for the workgroup's 16 channels: one row of
// 16 I/O words per token, padded by 8 bytes so that the 16 tokens a wave reads at once
// (one per lane of a row) fall in distinct banks.
template <class T>
constexpr int tok_pitch_bytes() { return kChannels * static_cast<int>(sizeof(T)) + 8; }

template <class T, int kStage>
struct Smem {
    static constexpr int kBPitch = kStage + 4;   // LDS pitch of one state's B column (floats)
    static constexpr int kTokPitch = tok_pitch_bytes<T>();
    static constexpr bool kCSwizzle = true;      // C rows in the swizzled token-row layout
    static constexpr bool kCCols = false;        // C as token rows (not columns)
    float bcol[2][kMaxState][kBPitch];           // [buffer][state][token]: B, transposed
    float crow[2][kStage][kPPitch];              // [buffer][token][state]: C rows
    float p[kWaves][kRowsPerWave * kRowPitch];   // [wave][row][token][state]: states h_t (padded)
    alignas(16) unsigned char tok[2][3][kStage][kTokPitch];  // [buffer][x|dt|z][token][channels]
};

// One B/C stage is 2 tensors x kStage tokens x 16 states.  kStagerThreads threads cover
// the 2*kStage (tensor, token) pairs with kParts threads per pair, each holding kPer
// states.  The raw words stay in registers while the current stage is computed and
// are converted to float32 when written to LDS.  Tokens past the end of the sequence
// re-load the last token (always in bounds); they only feed steps whose Delta is 0.
// kFullN: d_state == 16, rows of 16 states moved as 16-byte vectors.
template <class Io, int kStage, bool kFullN>
struct Stager {
    static constexpr int kPairs = 2 * kStage;               // (tensor, token) pairs per stage
    static constexpr int kParts = kStagerThreads / kPairs;    // threads per pair
    static constexpr int kPer = kMaxState / kParts;         // states per thread
    static_assert(kPairs * kParts == kStagerThreads && kPer * kParts == kMaxState, "stage shape");
    static constexpr int kWords = kPer * static_cast<int>(sizeof(typename Io::T)) / 16;  // uint4 words
    static_assert(!kFullN || kWords > 0, "16-byte rows");
    float v[kFullN ? 1 : kPer];
    uint4 w[kFullN ? kWords : 1];

    __device__ inline void load(const ScanArgs &a, size_t tbase, size_t t1, int N, int rtid)
    {
        const int pair = rtid / kParts;
        const int part = rtid % kParts;
        const int which = pair / kStage;
        const int tt = pair % kStage;
        size_t t = tbase + static_cast<size_t>(tt);
        if (t >= t1) t = t1 - 1;  // only called for non-empty sequences
        const void *src = which ? a.C : a.B;
        const int n0 = part * kPer;
        if constexpr (kFullN) {
            const uint4 *q =
                reinterpret_cast<const uint4 *>(static_cast<const typename Io::T *>(src) + t * kMaxState + n0);
#pragma unroll
            for (int k = 0; k < kWords; ++k) w[k] = q[k];
        } else {
#pragma unroll
            for (int k = 0; k < kPer; ++k) v[k] = (n0 + k) < N ? Io::ld(src, t * N + n0 + k) : 0.0f;
        }
    }

    // Pins the raw words to this point of the program: their conversion (in store) cannot
    // be hoisted up to the loads, where it would wait for the memory latency.
    __device__ inline void hold_raw()
    {
        if constexpr (kFullN) {
#pragma unroll
            for (int k = 0; k < kWords; ++k) hold(w[k]);
        } else {
#pragma unroll
            for (int k = 0; k < kPer; ++k) hold(v[k]);
        }
    }

    // LDS layout with bcol[2][kMaxState][>= kStage] and either (S::kCCols) C columns
    // ccol[2][kMaxState][>= kStage] or C rows crow[2][kStage][>= 16] (swizzled if S::kCSwizzle)
    template <class S>
    __device__ inline void store(S &sm, int buf, int rtid) const
    {
        const int pair = rtid / kParts;
        const int part = rtid % kParts;
        const int which = pair / kStage;
        const int tt = pair % kStage;
        const int n0 = part * kPer;
        float f[kPer];
        if constexpr (kFullN) {
            const uint32_t *u = reinterpret_cast<const uint32_t *>(w);
            if constexpr (sizeof(typename Io::T) == 2) {
#pragma unroll
                for (int k = 0; k < kPer / 2; ++k) {
                    f[2 * k] = bf16lo(u[k]);
                    f[2 * k + 1] = bf16hi(u[k]);
                }
            } else {
#pragma unroll
                for (int k = 0; k < kPer; ++k) f[k] = __uint_as_float(u[k]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < kPer; ++k) f[k] = v[k];
        }
        if (which == 0) {
            // B: transposed, one column per state (read by the lane that owns the state)
#pragma unroll
            for (int k = 0; k < kPer; ++k) sm.bcol[buf][n0 + k][tt] = f[k];
        } else if constexpr (S::kCCols) {
            // C: transposed like B (read by the lane that owns the state)
#pragma unroll
            for (int k = 0; k < kPer; ++k) sm.ccol[buf][n0 + k][tt] = f[k];
        } else {
            // C: token rows (read by the lane that finishes the token's readout)
#pragma unroll
            for (int k = 0; k < kPer / 4; ++k)
                *reinterpret_cast<float4 *>(
                    &sm.crow[buf][tt][S::kCSwizzle ? ((((n0 >> 2) + k) ^ tswz(tt)) << 2) : n0 + 4 * k]) =
                    make_float4(f[4 * k], f[4 * k + 1], f[4 * k + 2], f[4 * k + 3]);
        }
    }
};

// Token tiles of one stage: 3 tensors x kStage tokens x one 16-channel row (32 bytes for
// bf16, 64 for fp32), moved as 16-byte buffer loads (16-channel rows are
// contiguous in the token-major layout) and kept raw in registers until written to LDS.
// Tokens past the end of the sequence fall outside the resource's extent and load 0.
// Each tensor's resource is chosen at compile time (a resource picked from an array by a
// runtime index is not provably uniform and costs a waterfall loop per load).
template <class Io, int kStage>
struct TokStager {
    using T = typename Io::T;
    static constexpr int kRowBytes = kChannels * static_cast<int>(sizeof(T));
    static constexpr int kVecPerRow = kRowBytes / 16;
    static constexpr int kPerTensor = kStage * kVecPerRow;  // 16-byte vectors per tensor
    static constexpr int kPerThread = (kPerTensor + kStagerThreads - 1) / kStagerThreads;
    static_assert(kPerTensor % 64 == 0, "whole waves per vector slot");
    uint4 v[3][kPerThread];

    __device__ inline void load_one(Rsrc r, int k, int D, int c0, int rtid)
    {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int idx = i * kStagerThreads + rtid;
            if (kPerTensor % kStagerThreads == 0 || idx < kPerTensor) {  // uniform across each wave
                const int tok = idx / kVecPerRow;
                const int part = idx % kVecPerRow;
                const uint32_t boff = (static_cast<uint32_t>(tok) * static_cast<uint32_t>(D) + static_cast<uint32_t>(c0)) *
                                          static_cast<uint32_t>(sizeof(T)) +
                                      static_cast<uint32_t>(part * 16);
                v[k][i] = buf_ld128(r, boff);
            }
        }
    }

    __device__ inline void load(Rsrc rx, Rsrc rd, Rsrc rz, int D, int c0, int rtid)
    {
        load_one(rx, 0, D, c0, rtid);
        load_one(rd, 1, D, c0, rtid);
        load_one(rz, 2, D, c0, rtid);
    }

    template <class S>  // LDS layout with tok[2][3][kStage][>= 16 I/O words]
    __device__ inline void store(S &sm, int buf, int rtid) const
    {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const int idx = i * kStagerThreads + rtid;
                if (kPerTensor % kStagerThreads == 0 || idx < kPerTensor) {
                    const int tok = idx / kVecPerRow;
                    const int part = idx % kVecPerRow;
                    uint2 *d = reinterpret_cast<uint2 *>(&sm.tok[buf][k][tok][part * 16]);
                    d[0] = make_uint2(v[k][i].x, v[k][i].y);
                    d[1] = make_uint2(v[k][i].z, v[k][i].w);
                }
            }
        }
    }
};

}  // namespace rows

namespace rows {

constexpr int kLptMaxSeqs = 64;  // packed batches up to this many sequences run longest first

// Packed batches: the workgroups of a sequence take time in proportion to its length, and
// the hardware starts workgroups in index order, so the sequences are visited longest first
// (ties by index): a long sequence started last would otherwise run alone at the end.
// Returns the sequence of rank r in that order.  Every thread of the workgroup must call it
// (one barrier); nseq <= kLptMaxSeqs.
__device__ inline int longest_first(const ScanArgs &a, int r, int *order)
{
    const int t = threadIdx.x;
    if (t < a.nseq) {
        size_t b0, b1;
        seq_range(a, t, b0, b1);
        const size_t len = b1 - b0;
        int rank = 0;
        for (int u = 0; u < a.nseq; ++u) {
            size_t c0, c1;
            seq_range(a, u, c0, c1);
            const size_t lu = c1 - c0;
            rank += (lu > len || (lu == len && u < t)) ? 1 : 0;
        }
        order[rank] = t;
    }
    __syncthreads();
    return order[r];
}

}  // namespace rows

// kUIn: the x rows hold u = SiLU(conv(x)) already (the conv, its parameters and the
// history are not used).
template <class Io, int kStage, bool kFullN, bool kUIn>
__global__ __launch_bounds__(256) void rows_scan_kernel(ScanArgs a, int ncb)
{
    using namespace rows;
    using T = typename Io::T;
    constexpr int kStageBlocks = kStage / kBlock;
    __shared__ Smem<T, kStage> sm;
    __shared__ int seq_order[kLptMaxSeqs];

    // Workgroup -> (sequence, block of 16 channels); packed batches longest sequence first.
    const int bid = logical_block(blockIdx.x, gridDim.x);
    int s = bid / ncb;
    const int cb = bid - s * ncb;
    if (a.cu != nullptr && a.nseq > 1 && a.nseq <= kLptMaxSeqs) s = longest_first(a, s, seq_order);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int row = lane >> 4;
    const int j = lane & 15;           // state index n and token-in-block index
    const int D = a.D;
    const int N = a.N;
    const int c = cb * kChannels + wave * kRowsPerWave + row;
    const bool chan_ok = c < D;
    const int cc = chan_ok ? c : D - 1;  // clamped channel for loads; results discarded
    const bool state_ok = j < N;

    size_t t0, t1;
    seq_range(a, s, t0, t1);
    const int L = static_cast<int>(t1 - t0);

    const float An = state_ok ? a.A[static_cast<size_t>(cc) * N + j] : 0.0f;
    const float w0 = kUIn ? 0.0f : a.conv_w[cc * kConvK + 0], w1 = kUIn ? 0.0f : a.conv_w[cc * kConvK + 1];
    const float w2 = kUIn ? 0.0f : a.conv_w[cc * kConvK + 2], w3 = kUIn ? 0.0f : a.conv_w[cc * kConvK + 3];
    const float cbias = (!kUIn && a.conv_b) ? a.conv_b[cc] : 0.0f;
    const float dsk = a.Dskip ? a.Dskip[cc] : 0.0f;
    const float bias = a.dt_bias ? a.dt_bias[cc] : 0.0f;
    const size_t hidx = (static_cast<size_t>(s) * D + cc) * N + j;
    float h = (a.h0 != nullptr && state_ok) ? a.h0[hidx] : 0.0f;

    // History: lanes 13, 14, 15 of the "previous block" hold x_{t0-3}, x_{t0-2}, x_{t0-1}.
    // conv_final entry k receives x_{t1-3+k}: from the incoming history when t1-3+k < t0
    // (sequences shorter than 3 tokens), else from the sequence itself.  Every source is
    // read before any store, since conv_final may alias conv0.
    const size_t cbase = static_cast<size_t>(s) * 3 * D + cc;
    float xprev = 0.0f;
    if constexpr (!kUIn) {
        if (a.conv0 != nullptr && j >= 13) xprev = Io::ld(a.conv0, cbase + static_cast<size_t>(j - 13) * D);
        if (a.conv_final != nullptr && chan_ok && j >= 13) {
            const int k = j - 13;
            const int tk = L - 3 + k;  // token index relative to t0
            float hv;
            if (tk >= 0)
                hv = Io::ld(a.x, (t0 + static_cast<size_t>(tk)) * D + cc);
            else
                hv = (a.conv0 != nullptr) ? Io::ld(a.conv0, cbase + static_cast<size_t>(k + L) * D) : 0.0f;
            Io::st(a.conv_final, cbase + static_cast<size_t>(k) * D, hv);
        }
    }

    const int nstages = (L + kStage - 1) / kStage;
    const bool has_z = a.z != nullptr;
    const T *xs = static_cast<const T *>(a.x) + t0 * D;
    const T *dts = static_cast<const T *>(a.dt) + t0 * D;
    const T *zs = has_z ? static_cast<const T *>(a.z) + t0 * D : xs;
    T *os = static_cast<T *>(a.out) + t0 * D;

    // Byte extent of a stage's rows (the stage's tokens that belong to the sequence; only
    // stages that start inside it are addressed): buffer resources built on it bound every
    // token access of the stage.
    auto stage_bytes = [&](int base) {
        return static_cast<uint32_t>(min(kStage, L - base)) * static_cast<uint32_t>(D) * static_cast<uint32_t>(sizeof(T));
    };
    auto tok_off = [&](int tr) {  // byte offset of (token tr of a stage, this lane's channel)
        return (static_cast<uint32_t>(tr) * static_cast<uint32_t>(D) + static_cast<uint32_t>(cc)) *
               static_cast<uint32_t>(sizeof(T));
    };

    // Token tiles of one stage (x, dt, z for the workgroup's 16 channels).
    const int c0 = cb * kChannels;
    auto load_stage_tokens = [&](int st, TokStager<Io, kStage> &ts) {
        const int base = st * kStage;
        const uint32_t bytes = stage_bytes(base);
        const size_t off = static_cast<size_t>(base) * D;
        ts.load(make_rsrc(xs + off, bytes), make_rsrc(dts + off, bytes), make_rsrc(zs + off, bytes), D, c0, tid);
    };
    // This lane's channel within the workgroup's 16 (its column in the token tiles).
    const int lane_ch = wave * kRowsPerWave + row;

    // B column of one block for this lane's state, from the LDS stage buffer.
    struct Cols {
        float4 b[kBlock / 4];
    };
    auto read_cols = [&](int buf, int bk, Cols &cl) {
        const float *bcol = &sm.bcol[buf][j][bk * kBlock];
#pragma unroll
        for (int g = 0; g < kBlock / 4; ++g) cl.b[g] = *reinterpret_cast<const float4 *>(bcol + 4 * g);
    };

    float *pw = &sm.p[wave][row * kRowPitch];  // this row's 16x16 tile of states h_t[n]
    // Epilogue state of the block whose readout is in flight.
    float pu = 0.0f, pz = 0.0f;
    int pblk = -kBlock;  // its first token relative to t0 (negative: none yet)
    float4 py[kBlock / 4], pc[kBlock / 4];  // its token's 16 states and C row (lane j: token j)

    // Sum the transposed products of the in-flight block (already read into py), finish
    // its outputs and store them.  The store is unconditional: tokens past the end,
    // padding channels and the not-yet-existing block get an offset beyond the resource's
    // extent, which the hardware drops.  (A store inside a divergent branch makes the
    // compiler's vector-memory counter tracking give up and wait for every outstanding
    // store at the next use of loaded data.)
    auto finish = [&]() {
        // y = sum_n C_t[n] h_t[n] + D u_t  (four independent partial sums)
        float ya = pc[0].x * py[0].x, yb = pc[0].y * py[0].y, yc = pc[0].z * py[0].z, yd = pc[0].w * py[0].w;
#pragma unroll
        for (int g = 1; g < kBlock / 4; ++g) {
            ya = __builtin_fmaf(pc[g].x, py[g].x, ya);
            yb = __builtin_fmaf(pc[g].y, py[g].y, yb);
            yc = __builtin_fmaf(pc[g].z, py[g].z, yc);
            yd = __builtin_fmaf(pc[g].w, py[g].w, yd);
        }
        float y = (ya + yb) + (yc + yd);
        y = __builtin_fmaf(dsk, pu, y);
        const float o = has_z ? y * silu(pz) : y;
        const int ta = pblk + j;
        const int sb = max(pblk, 0) / kStage * kStage;
        const Rsrc ro = make_rsrc(os + static_cast<size_t>(sb) * D, stage_bytes(sb));
        const uint32_t boff = (pblk >= 0 && ta < L && chan_ok) ? tok_off(ta - sb) : 0xfffffff0u;
        buf_st(ro, boff, o, static_cast<T *>(nullptr));
    };
    // The in-flight block's states for this lane's token (transposed through the tile) and
    // its C row (from the stage buffer that held the block).
    auto read_products = [&]() {
        const float *pr = pw + j * kPPitch;
        const int cb_ = (max(pblk, 0) / kStage) & 1;
        const float *cr = &sm.crow[cb_][(max(pblk, 0) % kStage) + j][0];
#pragma unroll
        for (int g = 0; g < kBlock / 4; ++g) {
            const int q = (g ^ tswz(j)) << 2;  // token j's chunk g
            py[g] = *reinterpret_cast<const float4 *>(pr + q);
            pc[g] = *reinterpret_cast<const float4 *>(cr + q);
        }
    };
    // Raw token words of one block for this lane (read from the LDS tile one block ahead).
    struct TokRaw {
        T x, dt, z;
    };
    auto read_tok = [&](int buf, int bk, TokRaw &r) {
        const int tr = bk * kBlock + j;
        r.x = reinterpret_cast<const T *>(&sm.tok[buf][0][tr][0])[lane_ch];
        r.dt = reinterpret_cast<const T *>(&sm.tok[buf][1][tr][0])[lane_ch];
        r.z = reinterpret_cast<const T *>(&sm.tok[buf][2][tr][0])[lane_ch];
    };

    // Per-token front end of one block (lane j: token tb + j): causal conv with the taps
    // x_{t-1..t-3} from neighbouring lanes (row rotations), SiLU, softplus(dt + b) in log2
    // units, Delta * u.  Tokens past the end get Delta = 0 (the state does not move).
    struct Front {
        float x, u, zv, lg, du;
    };
    auto front = [&](const TokRaw &r, float xp, int tb, Front &f) {
        const bool act = tb + j < L;
        f.x = to_f32(r.x);
        f.zv = to_f32(r.z);
        if constexpr (kUIn) {
            f.u = f.x;
        } else {
            float pre = __builtin_fmaf(w3, f.x, cbias);
            pre = __builtin_fmaf(tap<1>(f.x, xp, j), w2, pre);
            pre = __builtin_fmaf(tap<2>(f.x, xp, j), w1, pre);
            pre = __builtin_fmaf(tap<3>(f.x, xp, j), w0, pre);
            f.u = silu(pre);
        }
        const float lg = softplus_log2(to_f32(r.dt) + bias);
        f.lg = act ? lg : 0.0f;
        f.du = act ? (lg * kLn2) * f.u : 0.0f;
    };

    Stager<Io, kStage, kFullN> stg;
    TokStager<Io, kStage> tst;
    Cols cl, cln;
    TokRaw tk1, tk2;  // token words of the next block and of the one after it
    Front fe, fen;    // front end of the current block and of the next one
    if (nstages > 0) {
        stg.load(a, t0, t1, N, tid);
        load_stage_tokens(0, tst);
        stg.store(sm, 0, tid);
        tst.store(sm, 0, tid);
    }
    __syncthreads();
    // Nothing loaded before the loop may still be in flight when it starts: otherwise the
    // compiler cannot tell those loads apart from the next stage's prefetch at the loop
    // header and waits for all of them at the first use.
    __builtin_amdgcn_s_waitcnt(0);

    for (int st = 0; st < nstages; ++st) {
        const int buf = st & 1;
        const bool more = st + 1 < nstages;
        const int sbase = st * kStage;
        // Stage prologue: B/C columns of block 0, token words of blocks 0 and 1, and the
        // front end of block 0 (the one front end per stage not overlapped with a recurrence).
        {
            TokRaw tk0;
            read_cols(buf, 0, cl);
            read_tok(buf, 0, tk0);
            read_tok(buf, 1, tk1);
            front(tk0, xprev, sbase, fe);
        }
        if (more) {
            stg.load(a, t0 + static_cast<size_t>(st + 1) * kStage, t1, N, tid);
            load_stage_tokens(st + 1, tst);
        }

        // Every block of the stage runs, also past the end of a short last stage: there
        // Delta is forced to 0 (the state does not move) and the stores are dropped.
        // Within one block: block bk's recurrence, block bk+1's front end and block
        // bk-1's readout are independent, so the scheduler can interleave them.
#pragma unroll
        for (int bk = 0; bk < kStageBlocks; ++bk) {
            const int tb = sbase + bk * kBlock;  // first token of the block (relative to t0)

            // ---- states and C row of the previous block: read now, consumed below
            wave_order();
            read_products();
            wave_order();
            // ---- LDS reads for the coming blocks (same stage buffer)
            if (bk + 1 < kStageBlocks) read_cols(buf, bk + 1, cln);
            if (bk + 2 < kStageBlocks) read_tok(buf, bk + 2, tk2);

            // ---- 16 recurrence steps; lane j holds state n = j.  First the 16 decay
            // factors exp(Delta_t A_n) and inputs Delta_t u_t B_t[n] (independent of the
            // state: 16 parallel chains), then the state chain itself (16 dependent FMAs).
            const float lg = fe.lg, du = fe.du;
            float ab[kBlock], bu[kBlock], p[kBlock];
#pragma unroll
            for (int g = 0; g < kBlock / 4; ++g) {
                const float bv[4] = {cl.b[g].x, cl.b[g].y, cl.b[g].z, cl.b[g].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * g + e;
                    float lt, dut;
                    switch (t) {
#define SAMBA_BCAST(k) case k: lt = dpp<kRowNewBcast + k>(lg); dut = dpp<kRowNewBcast + k>(du); break;
                        SAMBA_BCAST(0) SAMBA_BCAST(1) SAMBA_BCAST(2) SAMBA_BCAST(3)
                        SAMBA_BCAST(4) SAMBA_BCAST(5) SAMBA_BCAST(6) SAMBA_BCAST(7)
                        SAMBA_BCAST(8) SAMBA_BCAST(9) SAMBA_BCAST(10) SAMBA_BCAST(11)
                        SAMBA_BCAST(12) SAMBA_BCAST(13) SAMBA_BCAST(14) SAMBA_BCAST(15)
#undef SAMBA_BCAST
                    }
                    ab[t] = hw_exp2(lt * An);
                    bu[t] = dut * bv[e];
                }
            }
#pragma unroll
            for (int t = 0; t < kBlock; ++t) {
                h = __builtin_fmaf(ab[t], h, bu[t]);
                p[t] = h;
            }
            // ---- front end of the next block (its token words were read a block ago)
            if (bk + 1 < kStageBlocks) front(tk1, fe.x, tb + kBlock, fen);
            // ---- finish the previous block
            finish();

            // ---- publish this block's states (the tile was read above, in order)
            wave_order();
#pragma unroll
            for (int t = 0; t < kBlock; ++t) pw[t * kPPitch + row_elem(j, tswz(t))] = p[t];
            wave_order();

            pu = fe.u;
            pz = fe.zv;
            pblk = tb;
            xprev = fe.x;
            if (bk + 1 < kStageBlocks) {
                fe = fen;
                cl = cln;
                tk1 = tk2;
            }
        }

        if (more) {
            stg.store(sm, buf ^ 1, tid);
            tst.store(sm, buf ^ 1, tid);
        }
        __syncthreads();
    }

    // Finish the last block.
    if (nstages > 0) {
        wave_order();
        read_products();
        wave_order();
        finish();
    }
    if (a.h_final != nullptr && chan_ok && state_ok) a.h_final[hidx] = h;
}

// One wave per channel group, four waves per workgroup; used when the grid has enough
// workgroups for two or more waves per SIMD.  kStage 64 keeps two workgroups per CU.
inline void launch_rows_single(const ScanArgs &a, samba_dtype io, hipStream_t stream)
{
    const int ncb = (a.D + rows::kChannels - 1) / rows::kChannels;
    const dim3 grid(ncb * a.nseq), block(256);
    const bool full = a.N == kMaxState;
#define SAMBA_ROWS(IO, FULL, UIN) rows_scan_kernel<IO, 64, FULL, UIN><<<grid, block, 0, stream>>>(a, ncb)
    if (io == SAMBA_BF16) {
        if (a.u_in) {
            if (full) SAMBA_ROWS(IoBf16, true, true); else SAMBA_ROWS(IoBf16, false, true);
        } else {
            if (full) SAMBA_ROWS(IoBf16, true, false); else SAMBA_ROWS(IoBf16, false, false);
        }
    } else {
        if (a.u_in) {
            if (full) SAMBA_ROWS(IoF32, true, true); else SAMBA_ROWS(IoF32, false, true);
        } else {
            if (full) SAMBA_ROWS(IoF32, true, false); else SAMBA_ROWS(IoF32, false, false);
        }
    }
#undef SAMBA_ROWS
}

}  // namespace samba
