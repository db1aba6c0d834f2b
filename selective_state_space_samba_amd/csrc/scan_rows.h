// scan_rows.h -- prefill with one 16-lane DPP row per channel (one lane per state).
//
// The recurrence of page 1 section 3.4 ("The State Space Model Update (S6)") is
// independent across channels and, within a channel, across the d_state = 16 state
// components; only the readout y_t = sum_n C_t[n] h_t[n] couples the states.  This
// kernel therefore gives every channel a row of 16 lanes (lane n owns state n) and walks
// the sequence in time, so a batch-1 prompt of d_inner = 4096 channels still yields
// 65536 lanes with no cross-workgroup carry and no recomputation.
//
// Per block of 16 tokens, lane j of a row runs the per-token front end for token t0+j
// (causal conv with the taps x_{t-1..t-3} fetched from neighbouring lanes by DPP row
// rotations, SiLU, softplus(dt + b)), then all 16 lanes step their state through the 16
// tokens, receiving Delta and Delta*u of token t from lane t by DPP row broadcast fused
// into the multiply.  B and C of the block are staged once per workgroup into LDS as
// float32, transposed to [state][token], so each lane reads its state's column with
// 128-bit loads.  The 16 partial products C_t[n] h_t[n] of a lane are transposed through
// LDS so that lane j sums the readout of token t0+j, adds D*u, applies the SiLU(z) gate
// and stores the output.
#pragma once

#include "scan_common.h"

namespace samba {

namespace rows {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kRowsPerWave = 4;           // channels per wave (4 rows of 16 lanes)
constexpr int kChannels = kWaves * kRowsPerWave;  // channels per workgroup
constexpr int kBlock = 16;                // tokens per block (one per lane of a row)
constexpr int kStage = 64;                // tokens of B/C staged in LDS per stage
constexpr int kStageBlocks = kStage / kBlock;
constexpr int kBCPitch = kStage + 4;      // LDS pitch of one state's column (floats)
constexpr int kPPitch = kBlock + 4;       // LDS pitch of one token's 16 partial products

// DPP controls (gfx9 encoding).
constexpr int kRowRor = 0x120;      // row_ror:k = kRowRor + k  (k = 1..15)
constexpr int kRowNewBcast = 0x150; // row_newbcast:k = kRowNewBcast + k

template <int kCtrl>
__device__ inline float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, false));
}

// x_{t-s} for the lane's token: from lane j-s of this block, or lane 16+j-s of the previous
// block when j < s (row rotation of a per-lane select).
template <int kS>
__device__ inline float tap(float xcur, float xprev, int j)
{
    const float r = (j <= 15 - kS) ? xcur : xprev;
    return dpp<kRowRor + kS>(r);
}

struct Smem {
    float bc[2][2][kMaxState][kBCPitch];                        // [buffer][B|C][state][token]
    float p[kWaves][kRowsPerWave][kBlock][kPPitch];             // [wave][row][token][state]
};

// Loads (into registers) this thread's share of a B/C stage: 2 tensors x kStage tokens x 16
// states of bf16/f32.  Thread l handles tensor l/128, token (l%128)/2, states 8*(l%2)..+7.
template <class Io>
struct StageRegs {
    float v[8];
};

template <class Io>
__device__ inline void stage_load(const ScanArgs &a, size_t tbase, size_t t1, int N, int tid, StageRegs<Io> &r)
{
    const int which = tid >> 7;
    const int tt = (tid & 127) >> 1;
    const int n0 = (tid & 1) * 8;
    const size_t t = tbase + tt;
    const void *src = which ? a.C : a.B;
#pragma unroll
    for (int k = 0; k < 8; ++k) r.v[k] = 0.0f;
    if (t < t1) {
        if (N == kMaxState) {
            if constexpr (sizeof(typename Io::T) == 2) {
                const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + t * kMaxState + n0);
                r.v[0] = bf16lo(w.x); r.v[1] = bf16hi(w.x);
                r.v[2] = bf16lo(w.y); r.v[3] = bf16hi(w.y);
                r.v[4] = bf16lo(w.z); r.v[5] = bf16hi(w.z);
                r.v[6] = bf16lo(w.w); r.v[7] = bf16hi(w.w);
            } else {
                const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(src) + t * kMaxState + n0);
                const float4 u0 = p[0], u1 = p[1];
                r.v[0] = u0.x; r.v[1] = u0.y; r.v[2] = u0.z; r.v[3] = u0.w;
                r.v[4] = u1.x; r.v[5] = u1.y; r.v[6] = u1.z; r.v[7] = u1.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (n0 + k < N) r.v[k] = Io::ld(src, t * N + n0 + k);
        }
    }
}

template <class Io>
__device__ inline void stage_store(Smem &sm, int buf, int tid, const StageRegs<Io> &r)
{
    const int which = tid >> 7;
    const int tt = (tid & 127) >> 1;
    const int n0 = (tid & 1) * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) sm.bc[buf][which][n0 + k][tt] = r.v[k];
}

}  // namespace rows

template <class Io>
__global__ __launch_bounds__(256) void rows_scan_kernel(ScanArgs a, int ncb)
{
    using namespace rows;
    __shared__ Smem sm;

    // Workgroup -> (sequence, block of 16 channels).  Consecutive hardware workgroup ids
    // go round-robin to the 8 XCDs; remap so that each XCD gets a contiguous range of
    // channel blocks, and the 128-byte lines shared by 4 neighbouring blocks meet in
    // one L2.
    const int nb = gridDim.x;
    const int q = nb >> 3;
    int bid = blockIdx.x;
    if (bid < (q << 3)) bid = (bid & 7) * q + (bid >> 3);
    const int s = bid / ncb;
    const int cb = bid - s * ncb;

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

    const float An = state_ok ? a.A[static_cast<size_t>(cc) * N + j] : 0.0f;
    const float w0 = a.conv_w[cc * kConvK + 0], w1 = a.conv_w[cc * kConvK + 1];
    const float w2 = a.conv_w[cc * kConvK + 2], w3 = a.conv_w[cc * kConvK + 3];
    const float cbias = a.conv_b ? a.conv_b[cc] : 0.0f;
    const float dsk = a.Dskip ? a.Dskip[cc] : 0.0f;
    const float bias = a.dt_bias ? a.dt_bias[cc] : 0.0f;
    const size_t hidx = (static_cast<size_t>(s) * D + cc) * N + j;
    float h = (a.h0 != nullptr && state_ok) ? a.h0[hidx] : 0.0f;

    // History: lanes 13, 14, 15 of the "previous block" hold x_{t0-3}, x_{t0-2}, x_{t0-1}.
    const size_t cbase = static_cast<size_t>(s) * 3 * D + cc;
    float xprev = 0.0f;
    if (a.conv0 != nullptr && j >= 13) xprev = Io::ld(a.conv0, cbase + static_cast<size_t>(j - 13) * D);
    // conv_final entries that lie before t0 (sequences shorter than 3 tokens): copy the
    // tail of the incoming history (read above, before any store can overwrite it).
    const size_t L = t1 - t0;
    if (a.conv_final != nullptr && chan_ok && L < 3 && j >= 13 && j - 13 + static_cast<int>(L) <= 2) {
        // entry k = j - 13 receives x_{t1-3+k} = history entry k + L
        const int k = j - 13;
        const float hv = (a.conv0 != nullptr) ? Io::ld(a.conv0, cbase + static_cast<size_t>(k + L) * D) : 0.0f;
        Io::st(a.conv_final, cbase + static_cast<size_t>(k) * D, hv);
    }

    const size_t nblocks = (L + kBlock - 1) / kBlock;
    const size_t nstages = (nblocks + kStageBlocks - 1) / kStageBlocks;

    // Prologue: stage 0 of B/C into LDS buffer 0.
    StageRegs<Io> sr;
    if (nstages > 0) {
        stage_load<Io>(a, t0, t1, N, tid, sr);
        stage_store<Io>(sm, 0, tid, sr);
    }
    __syncthreads();

    // Per-token inputs of the first block.
    auto load_tok = [&](size_t tb, float &xv, float &dtv, float &zv) {
        const size_t t = tb + j;
        xv = dtv = zv = 0.0f;
        if (t < t1) {
            const size_t ix = t * D + cc;
            xv = Io::ld(a.x, ix);
            dtv = Io::ld(a.dt, ix);
            zv = a.z ? Io::ld(a.z, ix) : 0.0f;
        }
    };
    float xn, dtn, zn;
    if (nblocks > 0) load_tok(t0, xn, dtn, zn);

    float *pw = &sm.p[wave][row][0][0];

    for (size_t st = 0; st < nstages; ++st) {
        const int buf = static_cast<int>(st & 1);
        const bool more = st + 1 < nstages;
        if (more) stage_load<Io>(a, t0 + (st + 1) * kStage, t1, N, tid, sr);

        for (int bk = 0; bk < kStageBlocks; ++bk) {
            const size_t blk = st * kStageBlocks + bk;
            if (blk >= nblocks) break;  // uniform across the workgroup
            const size_t tb = t0 + blk * kBlock;
            const float xv = xn, dtv = dtn, zv = zn;
            if (blk + 1 < nblocks) load_tok(tb + kBlock, xn, dtn, zn);
            const bool act = tb + j < t1;

            // ---- front end for token tb + j: conv taps, SiLU, softplus
            float pre = __builtin_fmaf(w3, xv, cbias);
            pre = __builtin_fmaf(w2, tap<1>(xv, xprev, j), pre);
            pre = __builtin_fmaf(w1, tap<2>(xv, xprev, j), pre);
            pre = __builtin_fmaf(w0, tap<3>(xv, xprev, j), pre);
            const float u = silu(pre);
            float lg = softplus_log2(dtv + bias);
            lg = act ? lg : 0.0f;
            const float du = act ? (lg * kLn2) * u : 0.0f;

            // ---- 16 recurrence steps; lane j holds state n = j
            const float *bcol = &sm.bc[buf][0][j][bk * kBlock];
            const float *ccol = &sm.bc[buf][1][j][bk * kBlock];
            float p[kBlock];
#pragma unroll
            for (int g = 0; g < kBlock / 4; ++g) {
                const float4 bq = *reinterpret_cast<const float4 *>(bcol + 4 * g);
                const float4 cq = *reinterpret_cast<const float4 *>(ccol + 4 * g);
                const float bv[4] = {bq.x, bq.y, bq.z, bq.w};
                const float cv[4] = {cq.x, cq.y, cq.z, cq.w};
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
                    const float ab = hw_exp2(lt * An);
                    h = __builtin_fmaf(ab, h, dut * bv[e]);
                    p[t] = cv[e] * h;
                }
            }

            // ---- readout: transpose the 16x16 partial products of the row through LDS
#pragma unroll
            for (int t = 0; t < kBlock; ++t) pw[t * kPPitch + j] = p[t];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const float *pr = pw + j * kPPitch;
            float y = 0.0f;
#pragma unroll
            for (int g = 0; g < kBlock / 4; ++g) {
                const float4 v = *reinterpret_cast<const float4 *>(pr + 4 * g);
                y += (v.x + v.y) + (v.z + v.w);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            y = __builtin_fmaf(dsk, u, y);
            const float o = a.z ? y * silu(zv) : y;
            if (act && chan_ok) {
                const size_t t = tb + j;
                Io::st(a.out, t * D + cc, o);
                if (a.conv_final != nullptr && t + 3 >= t1) Io::st(a.conv_final, cbase + (t + 3 - t1) * D, xv);
            }
            xprev = xv;
        }

        if (more) stage_store<Io>(sm, buf ^ 1, tid, sr);
        __syncthreads();
    }

    if (a.h_final != nullptr && chan_ok && state_ok) a.h_final[hidx] = h;
}

inline void launch_rows_scan(const ScanArgs &a, samba_dtype io, hipStream_t stream)
{
    const int ncb = (a.D + rows::kChannels - 1) / rows::kChannels;
    const dim3 grid(ncb * a.nseq), block(256);
    if (io == SAMBA_BF16)
        rows_scan_kernel<IoBf16><<<grid, block, 0, stream>>>(a, ncb);
    else
        rows_scan_kernel<IoF32><<<grid, block, 0, stream>>>(a, ncb);
}

}  // namespace samba
