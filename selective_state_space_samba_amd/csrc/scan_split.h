// scan_split.h -- prefill with one 16-lane DPP row per channel (one lane per state), the
// work of every channel split between two waves of different roles.
//
// The recurrence of page 1 section 3.4 ("The State Space Model Update (S6)") is
// independent across channels and, within a channel, across the d_state = 16 state
// components; only the readout y_t = sum_n C_t[n] h_t[n] couples the states.  This
// kernel therefore gives every channel a row of 16 lanes (lane n owns state n) and walks
// the sequence in time, so a batch-1 prompt of d_inner = 4096 channels still yields
// 65536 lanes with no cross-workgroup carry and no recomputation.
//
// 65536 lanes are one wave per SIMD, and a single wave issues at most one instruction per
// issue cycle of its SIMD: its LDS, scalar and memory instructions would each cost a
// VALU slot.  So every channel gets two waves on the same SIMD, one per role:
//  * the token wave (lane j of a row = token j of a block of 16) runs the per-token work:
//    causal conv (taps from neighbouring lanes by DPP row rotations), SiLU,
//    softplus(dt + b), Delta and Delta*u, which it hands to the scan wave through LDS;
//    and the readout of a finished block (C_t . h_t + D u_t, SiLU(z) gate, store);
//  * the scan wave (lane n of a row = state n) steps the 16 states through the block,
//    receiving Delta and Delta*u of token t from lane t by DPP row broadcast fused into
//    the multiply, and writes the 16x16 tile of states h_t[n] to LDS (lane n: its 16
//    tokens as four 16-byte writes), where the token wave reads it transposed (lane j:
//    token j's 16 states, 16 four-byte reads).
// Both roles of a workgroup advance in lockstep, one 16-token block per step and one
// workgroup barrier per step: at step k the scan waves run block k while the token waves
// run the front end of block k+2 and the readout of block k-1.  The VALU work of the two
// roles then shares the SIMD while each role's LDS / memory / scalar instructions and
// stalls are covered by the other role.
//
// Per stage of kStage tokens the token waves stage B and C (shared by the workgroup's 16
// channels) into LDS as float32 (B transposed to [state][token], C as token rows) and the
// x / dt / z rows of the 16 channels (16-byte buffer loads), both into the other half of
// double buffers, with the loads issued one stage ahead.
//
// With a precomputed u (kUIn: u = SiLU(conv(x)) from samba_conv_silu, the activation a
// full layer also feeds to x_proj), the token rows carry u instead of x and the conv is
// skipped.
#pragma once

#include "scan_rows.h"

namespace samba {

namespace split {

constexpr int kRoleWaves = 4;                                  // waves per role
constexpr int kRoleThreads = kRoleWaves * 64;                  // threads per role
constexpr int kThreads = 2 * kRoleThreads;                     // threads per workgroup
constexpr int kExSlots = 4;                                    // Delta hand-over slots (blocks in flight)
constexpr int kMaxSplitGrid = 256;                             // workgroups: one per CU
static_assert(kRoleWaves * rows::kRowsPerWave == rows::kChannels && kRoleThreads == rows::kStagerThreads,
              "roles cover the 16 channels of a workgroup");
// State tiles keep one 80-byte row per state (16 tokens + 4 floats of padding) in 336-float
// channel tiles: a scan lane writes its state's 16 tokens as four 16-byte writes and a token
// lane reads its token's 16 states as 16 four-byte reads, both free of bank conflicts.  The
// other orientation (token rows: 16 four-byte writes per scan lane, four 16-byte reads per
// token lane) measured 2.5 % slower: it puts the larger instruction count on the scan waves,
// the critical path.  C rows keep 80-byte token rows (16 states + 4 floats of padding).
constexpr int kSPPitch = rows::kBlock + 4;
constexpr int kSRowPitch = rows::kBlock * kSPPitch + 16;

template <class T, int kStage, int kHsSlots>
struct SplitSmem {
    static constexpr int kBPitch = kStage + 4;   // LDS pitch of one state's B column (floats)
    static constexpr int kTokPitch = rows::tok_pitch_bytes<T>();
    float bcol[2][kMaxState][kBPitch];           // [buffer][state][token]: B, transposed
    static constexpr bool kCSwizzle = false;     // C rows unswizzled (see kSPPitch)
    static constexpr bool kCCols = false;        // C as token rows (read by the token role)
    float crow[2][kStage][kSPPitch];             // [buffer][token][state]: C rows
    float hs[kHsSlots][rows::kChannels * kSRowPitch];  // [block slot][channel][state][token]: h_t
    float lg[kExSlots][rows::kChannels * rows::kBlock];  // [slot][channel][token]: Delta * log2(e)
    float du[kExSlots][rows::kChannels * rows::kBlock];  // [slot][channel][token]: Delta * u
    alignas(16) unsigned char tok[2][3][kStage][kTokPitch];  // [buffer][x|dt|z][token][channels]
};

}  // namespace split

template <class Io, int kStage, bool kFullN, int kDist, bool kUIn>
__global__ __launch_bounds__(split::kThreads) void rows_split_kernel(ScanArgs a, int ncb)
{
    using namespace rows;
    using namespace split;
    using T = typename Io::T;
    constexpr int kSB = kStage / kBlock;  // blocks (steps) per stage
    // Hand-over distance: a value written in step k is read in step k + kDist, and the
    // workgroup barrier runs after every kDist-th step (after steps kDist-1, 2 kDist-1, ...),
    // so exactly one barrier lies between every write and its read.  At step k the scan
    // role runs block k (its Delta and B columns were read in step k-1) and publishes block
    // k-1's states; the token role computes the front end of block k+1+kDist (from token
    // words read in step k-1) and reads out block k-1-kDist.  State tiles live in 2 kDist
    // slots, so that no tile is rewritten before a barrier has passed after its last read.
    constexpr int kHsSlots = 2 * kDist;
    // The token role stages the data of stage s+1 during stage s.  Token words are first
    // read (a step ahead) at step kSB-2-kDist; they are written at the last step before the
    // barrier preceding that (their buffer's previous contents were last read in stage s-1).
    // B columns and C rows are written later, spreading the LDS writes: after a barrier
    // that follows the last readout of stage s-1's C rows (step kDist) and before the
    // barrier preceding the first read of the new B columns (step kSB-1).
    constexpr int kStoreStep = ((kSB - 2 - kDist) / kDist) * kDist - 1;
    constexpr int kStoreStepBC = ((kSB - 1) / kDist) * kDist - 1;
    static_assert(kDist == 1 || kDist == 2, "hand-over distance");
    static_assert(kSB >= 8 && kSB % kExSlots == 0 && kSB % kDist == 0, "stage length");
    static_assert(kStoreStep >= 0 && kStoreStepBC >= 2 * kDist && kStoreStepBC >= kStoreStep, "stage store steps");
    __shared__ SplitSmem<T, kStage, kHsSlots> sm;
    auto step_barrier = [](int bk) {
        if (bk % kDist == kDist - 1) __syncthreads();
    };

    // Workgroup -> (sequence, block of 16 channels).
    const int bid = logical_block(blockIdx.x, gridDim.x);
    const int s = bid / ncb;
    const int cb = bid - s * ncb;

    const int tid = threadIdx.x;
    // Role of the wave: uniform, so the role branch is a scalar branch; both roles pass
    // the same sequence of workgroup barriers.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool scan_role = wave >= kRoleWaves;
    const int rtid = tid & (kRoleThreads - 1);  // thread index within the role
    const int lane = tid & 63;
    const int row = lane >> 4;
    const int j = lane & 15;  // state n (scan role) or token of the block (token role)
    const int ch = (wave & (kRoleWaves - 1)) * kRowsPerWave + row;  // channel within the workgroup
    const int D = a.D;
    const int N = a.N;
    const int c = cb * kChannels + ch;
    const bool chan_ok = c < D;
    const int cc = chan_ok ? c : D - 1;  // clamped channel for loads; results discarded

    size_t t0, t1;
    seq_range(a, s, t0, t1);
    const int L = static_cast<int>(t1 - t0);
    const int nstages = (L + kStage - 1) / kStage;
    const int c0 = cb * kChannels;

    if (scan_role) {
        // ================================================================ scan role
        const bool state_ok = j < N;
        const float An = state_ok ? a.A[static_cast<size_t>(cc) * N + j] : 0.0f;
        const size_t hidx = (static_cast<size_t>(s) * D + cc) * N + j;
        float h = (a.h0 != nullptr && state_ok) ? a.h0[hidx] : 0.0f;
        float *hw = &sm.hs[0][ch * kSRowPitch + j * kSPPitch];  // this lane's state row of the tile

        struct Cols {
            float4 b[kBlock / 4];
        };
        auto read_cols = [&](int buf, int bk, Cols &cl) {
            const float *bcol = &sm.bcol[buf][j][bk * kBlock];
#pragma unroll
            for (int g = 0; g < kBlock / 4; ++g) cl.b[g] = *reinterpret_cast<const float4 *>(bcol + 4 * g);
        };

        __syncthreads();  // stage 0 in LDS
        __syncthreads();  // Delta of blocks 0 .. kDist published
        // Delta, Delta*u (lane n: token n) and B columns of the block about to run.
        float lgc = sm.lg[0][ch * kBlock + j], duc = sm.du[0][ch * kBlock + j];
        Cols cl;
        read_cols(0, 0, cl);

        // States of the previous block, published at the start of the next step (so that
        // the step's barrier never waits for fresh stores).
        float pp[kBlock];
#pragma unroll
        for (int t = 0; t < kBlock; ++t) pp[t] = 0.0f;
        for (int st = 0; st < nstages; ++st) {
            const int buf = st & 1;
#pragma unroll
            for (int bk = 0; bk < kSB; ++bk) {
                // ---- publish block k-1 (its slot; zeros before block 0)
                {
                    float *hp = hw + ((bk + kHsSlots - 1) % kHsSlots) * (kChannels * kSRowPitch);
#pragma unroll
                    for (int g = 0; g < kBlock / 4; ++g)
                        *reinterpret_cast<float4 *>(hp + 4 * g) = make_float4(pp[4 * g], pp[4 * g + 1], pp[4 * g + 2], pp[4 * g + 3]);
                }
                // ---- next block's inputs (published by the token role kDist steps ago)
                const int nslot = (bk + 1) % kExSlots;
                const float lgn = sm.lg[nslot][ch * kBlock + j], dun = sm.du[nslot][ch * kBlock + j];
                Cols cln;
                if (bk + 1 < kSB)
                    read_cols(buf, bk + 1, cln);
                else
                    read_cols(buf ^ 1, 0, cln);
                // keep the LDS traffic at the top of the step
                __builtin_amdgcn_sched_barrier(0);

                // ---- 16 recurrence steps; lane j holds state n = j.  First the 16 decay
                // factors exp(Delta_t A_n) and inputs Delta_t u_t B_t[n] (independent of the
                // state: 16 parallel chains), then the state chain itself (16 dependent FMAs).
                float ab[kBlock], bu[kBlock];
#pragma unroll
                for (int g = 0; g < kBlock / 4; ++g) {
                    const float bv[4] = {cl.b[g].x, cl.b[g].y, cl.b[g].z, cl.b[g].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 4 * g + e;
                        float lt, dut;
                        switch (t) {
#define SAMBA_BCAST(k) case k: lt = dpp<kRowNewBcast + k>(lgc); dut = dpp<kRowNewBcast + k>(duc); break;
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
                    pp[t] = h;
                }
                step_barrier(bk);
                lgc = lgn;
                duc = dun;
                cl = cln;
                hold(lgc);
                hold(duc);
#pragma unroll
                for (int g = 0; g < kBlock / 4; ++g) hold(cl.b[g]);
            }
        }
        // Publish the last block.
        if (nstages > 0) {
            float *hp = hw + ((nstages * kSB - 1) % kHsSlots) * (kChannels * kSRowPitch);
#pragma unroll
            for (int g = 0; g < kBlock / 4; ++g)
                *reinterpret_cast<float4 *>(hp + 4 * g) = make_float4(pp[4 * g], pp[4 * g + 1], pp[4 * g + 2], pp[4 * g + 3]);
        }
        __syncthreads();
        if (a.h_final != nullptr && chan_ok && state_ok) a.h_final[hidx] = h;
        return;
    }

    // ==================================================================== token role
    const float w0 = kUIn ? 0.0f : a.conv_w[cc * kConvK + 0], w1 = kUIn ? 0.0f : a.conv_w[cc * kConvK + 1];
    const float w2 = kUIn ? 0.0f : a.conv_w[cc * kConvK + 2], w3 = kUIn ? 0.0f : a.conv_w[cc * kConvK + 3];
    const float cbias = (!kUIn && a.conv_b) ? a.conv_b[cc] : 0.0f;
    const float dsk = a.Dskip ? a.Dskip[cc] : 0.0f;
    const float bias = a.dt_bias ? a.dt_bias[cc] : 0.0f;

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

    const bool has_z = a.z != nullptr;
    const T *xs = static_cast<const T *>(a.x) + t0 * D;
    const T *dts = static_cast<const T *>(a.dt) + t0 * D;
    const T *zs = has_z ? static_cast<const T *>(a.z) + t0 * D : xs;
    T *os = static_cast<T *>(a.out) + t0 * D;

    // Byte extent of a stage's rows (the stage's tokens that belong to the sequence; 0 for
    // a stage past the end): buffer resources built on it bound every token access.
    auto stage_bytes = [&](int base) {
        return static_cast<uint32_t>(max(0, min(kStage, L - base))) * static_cast<uint32_t>(D) *
               static_cast<uint32_t>(sizeof(T));
    };
    auto tok_off = [&](int tr) {  // byte offset of (token tr of a stage, this lane's channel)
        return (static_cast<uint32_t>(tr) * static_cast<uint32_t>(D) + static_cast<uint32_t>(cc)) *
               static_cast<uint32_t>(sizeof(T));
    };
    TokStager<Io, kStage> tst;
    auto load_stage_tokens = [&](int st) {
        const int base = st * kStage;
        const uint32_t bytes = stage_bytes(base);
        const size_t off = static_cast<size_t>(min(base, L)) * D;
        tst.load(make_rsrc(xs + off, bytes), make_rsrc(dts + off, bytes), make_rsrc(zs + off, bytes), D, c0, rtid);
    };

    // Raw token words of one block for this lane (token j of the block, channel ch).
    struct TokRaw {
        T x, dt, z;
    };
    auto read_tok = [&](int buf, int bk, TokRaw &r) {
        const int tr = bk * kBlock + j;
        r.x = reinterpret_cast<const T *>(&sm.tok[buf][0][tr][0])[ch];
        r.dt = reinterpret_cast<const T *>(&sm.tok[buf][1][tr][0])[ch];
        r.z = reinterpret_cast<const T *>(&sm.tok[buf][2][tr][0])[ch];
    };
    // Per-token front end of one block (lane j: token tb + j): causal conv with the taps
    // x_{t-1..t-3} from neighbouring lanes (row rotations), SiLU, softplus(dt + b) in log2
    // units and Delta * u, published to the scan role.  Tokens past the end get Delta = 0
    // (the state does not move).
    struct Front {
        float x, u, zv;
    };
    auto front = [&](const TokRaw &r, float xp, int tb, int slot, Front &f) {
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
        sm.lg[slot][ch * kBlock + j] = act ? lg : 0.0f;
        sm.du[slot][ch * kBlock + j] = act ? (lg * kLn2) * f.u : 0.0f;
    };
    // Readout of the block whose first token is pb (relative to t0; negative: none): lane j
    // sums token j's 16 states against its C row, adds D*u, gates and stores.  The store is
    // unconditional: tokens past the end, padding channels and the not-yet-existing block
    // get an offset beyond the resource's extent, which the hardware drops.
    auto finish = [&](const float4 *py, const float4 *pc, float pu, float pz, int pb) {
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
        const int ta = pb + j;
        const int sb = max(pb, 0) / kStage * kStage;
        const Rsrc ro = make_rsrc(os + static_cast<size_t>(sb) * D, stage_bytes(sb));
        const uint32_t boff = (pb >= 0 && ta < L && chan_ok) ? tok_off(ta - sb) : 0xfffffff0u;
        buf_st(ro, boff, o, static_cast<T *>(nullptr));
    };
    // A finished block's states for this lane's token (tile slot hslot) and the token's C
    // row (block cbk of stage buffer cbuf).
    const float *hr = &sm.hs[0][ch * kSRowPitch + j];
    auto read_states = [&](int hslot, int cbuf, int cbk, float4 *py, float4 *pc) {
        const float *pr = hr + hslot * (kChannels * kSRowPitch);
        const float *cr = &sm.crow[cbuf][cbk * kBlock + j][0];
#pragma unroll
        for (int g = 0; g < kBlock / 4; ++g) {
            py[g] = make_float4(pr[(4 * g) * kSPPitch], pr[(4 * g + 1) * kSPPitch], pr[(4 * g + 2) * kSPPitch],
                                pr[(4 * g + 3) * kSPPitch]);
            pc[g] = *reinterpret_cast<const float4 *>(cr + 4 * g);
        }
    };

    Stager<Io, kStage, kFullN> stg;
    if (nstages > 0) {
        stg.load(a, t0, t1, N, rtid);
        load_stage_tokens(0);
        stg.hold_raw();
        stg.store(sm, 0, rtid);
        tst.store(sm, 0, rtid);
    }
    __syncthreads();  // stage 0 in LDS
    // Fronts of the blocks in flight, fr[i] = block k-1-kDist+i at step k: fr[0] is read out,
    // fr[2 kDist + 2] is computed (from token words rn, read a step ahead).
    constexpr int kFronts = 2 * kDist + 3;
    Front fr[kFronts] = {};
    TokRaw rn;
    {
        TokRaw r;
        float xp = xprev;
#pragma unroll
        for (int m = 0; m <= kDist; ++m) {
            read_tok(0, m, r);
            front(r, xp, m * kBlock, m, fr[kDist + 1 + m]);
            xp = fr[kDist + 1 + m].x;
        }
        read_tok(0, kDist + 1, rn);
    }
    __syncthreads();  // Delta of blocks 0 .. kDist published

    for (int st = 0; st < nstages; ++st) {
        const int buf = st & 1;
        const int sbase = st * kStage;
        // Next stage's token words (past the last stage: empty extent, the loads return 0)
        // and B/C rows (past the last stage: clamped re-loads, never used).
        load_stage_tokens(st + 1);
        stg.load(a, t0 + static_cast<size_t>(st + 1) * kStage, t1, N, rtid);
#pragma unroll
        for (int bk = 0; bk < kSB; ++bk) {
            const int tb = sbase + bk * kBlock;  // first token of block k (relative to t0)
            // ---- LDS reads: states and C row of block k-1-kDist (published at step
            // k-kDist), token words of block k+2+kDist
            constexpr int kLag = 1 + kDist;
            float4 py[kBlock / 4], pc[kBlock / 4];
            const int hslot = (bk + kHsSlots * 2 - kLag) % kHsSlots;
            if (bk >= kLag)
                read_states(hslot, buf, bk - kLag, py, pc);
            else
                read_states(hslot, buf ^ 1, kSB + bk - kLag, py, pc);
            TokRaw r3;
            if (bk + kLag + 1 < kSB)
                read_tok(buf, bk + kLag + 1, r3);
            else
                read_tok(buf ^ 1, bk + kLag + 1 - kSB, r3);
            __builtin_amdgcn_sched_barrier(0);  // issue the reads before the arithmetic
            // ---- front end of block k+1+kDist, published for the scan role
            front(rn, fr[kFronts - 2].x, tb + kLag * kBlock, (bk + kLag) % kExSlots, fr[kFronts - 1]);
            // ---- readout of block k-1-kDist (after the front end, which covers the reads'
            // latency)
            __builtin_amdgcn_sched_barrier(0);
            finish(py, pc, fr[0].u, fr[0].zv, tb - kLag * kBlock);
            if (bk == kStoreStep) tst.store(sm, buf ^ 1, rtid);
            if (bk == kStoreStepBC) {
                stg.hold_raw();
                stg.store(sm, buf ^ 1, rtid);
            }
            step_barrier(bk);
#pragma unroll
            for (int i = 0; i + 1 < kFronts; ++i) fr[i] = fr[i + 1];
            rn = r3;
            hold(rn.x);
            hold(rn.dt);
            hold(rn.z);
        }
    }
    // Readout of the last 1 + kDist blocks: all but the last were published in the loop,
    // the last one after it.
    if (nstages > 0) {
        const int nb = nstages * kSB;
        const int lbuf = (nstages - 1) & 1;
#pragma unroll
        for (int i = 0; i < kDist; ++i) {
            const int m = nb - 1 - kDist + i;
            float4 py[kBlock / 4], pc[kBlock / 4];
            read_states(m % kHsSlots, lbuf, kSB - 1 - kDist + i, py, pc);
            finish(py, pc, fr[i].u, fr[i].zv, m * kBlock);
        }
    }
    __syncthreads();
    if (nstages > 0) {
        const int nb = nstages * kSB;
        float4 py[kBlock / 4], pc[kBlock / 4];
        read_states((nb - 1) % kHsSlots, (nstages - 1) & 1, kSB - 1, py, pc);
        finish(py, pc, fr[kDist].u, fr[kDist].zv, (nb - 1) * kBlock);
    }
}

inline void launch_rows_split(const ScanArgs &a, samba_dtype io, hipStream_t stream)
{
    const int ncb = (a.D + rows::kChannels - 1) / rows::kChannels;
    const dim3 grid(ncb * a.nseq), block(split::kThreads);
    const bool full = a.N == kMaxState;
    // Hand-over distance 2 (a barrier every other step) needs 4 state-tile slots, which fit
    // next to the 2-byte token tiles; with 4-byte token tiles the kernel syncs every step.
#define SAMBA_SPLIT(IO, FULL, DIST, UIN) rows_split_kernel<IO, 128, FULL, DIST, UIN><<<grid, block, 0, stream>>>(a, ncb)
    if (io == SAMBA_BF16) {
        if (a.u_in) {
            if (full) SAMBA_SPLIT(IoBf16, true, 2, true); else SAMBA_SPLIT(IoBf16, false, 2, true);
        } else {
            if (full) SAMBA_SPLIT(IoBf16, true, 2, false); else SAMBA_SPLIT(IoBf16, false, 2, false);
        }
    } else {
        if (a.u_in) {
            if (full) SAMBA_SPLIT(IoF32, true, 1, true); else SAMBA_SPLIT(IoF32, false, 1, true);
        } else {
            if (full) SAMBA_SPLIT(IoF32, true, 1, false); else SAMBA_SPLIT(IoF32, false, 1, false);
        }
    }
#undef SAMBA_SPLIT
}

}  // namespace samba
