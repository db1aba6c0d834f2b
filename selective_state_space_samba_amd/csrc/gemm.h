// gemm.h -- bfloat16 matrix-core GEMM for the projections of a Samba layer (gfx950).
//
// out = A . W^T with A [M, K] (token rows) and W [N, K] (one row per output feature, the
// transpose of the pages' d_in x d_out projection matrices), fp32 accumulation on
// v_mfma_f32_16x16x32_bf16.  Epilogues fused into the store:
//   store   out bf16 [M, ldo]                 (in_proj, gate, x_proj, dt, q/k/v)
//   add     out fp32 = residual fp32 + A.W^T  (the residual stream after W_out, W_o, W_3)
//   swiglu  W = [W1; W2] (2N rows), out bf16 = (A.W1^T) * SiLU(A.W2^T)
//           (page "Samba: Simple Hybrid State Space Models ...", "SwiGLU Formulation")
//
// Tiling.  A workgroup of WGM x WGN waves computes a TM x TN tile, TM = 16 FM WGM,
// TN = 16 FN WGN; each wave a 16FM x 16FN block of 16 x 16 MFMA tiles.  K advances 64 at a
// time through double-buffered LDS tiles (swizzled 128-byte rows, see kPitch); the next K
// tile's global loads are in flight while the current one is multiplied.  256 x 256 tiles
// run on 8 waves (4 x 2, 64 x 128 per wave, two waves per SIMD) with the operands loaded
// straight into LDS (gemm_ring_kernel); 128 x 128 tiles on 4 waves (2 x 2, two workgroups
// per CU) with loads staged through registers (gemm_kernel).  MFMA operand layouts (16x16x32 bf16):
// lane l supplies A[i = l % 16][k = 8 (l / 16) + e] and B[k = 8 (l / 16) + e][j = l % 16],
// e = 0..7, and receives D[i = 4 (l / 16) + e][j = l % 16], e = 0..3.  Both operands are
// K-contiguous rows (A rows, W rows), so both fragments are one 16-byte LDS read.
//
// Split K.  When the tiles alone cannot fill the chip (decode: M = a few hundred rows),
// the K range is cut into splits that write fp32 partial tiles to a workspace; a second
// kernel sums the splits in a fixed order (deterministic) and applies the epilogue.
#pragma once

#include "scan_common.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace samba {
namespace gemm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kTK = 64;          // K per LDS stage
// LDS tiles: 128-byte rows (kTK elements, unpadded), 16-byte chunk q of row r stored at chunk
// q ^ ((r >> 1) & 7).  Measured with rocprofv3 on gfx950: 16-byte reads of 16 rows at one
// chunk spend half their LDS cycles in bank conflicts with a padded 144-byte pitch and none
// with this swizzle; the staging writes (8 lanes per row) are conflict-free either way.
constexpr int kPitch = kTK;
__device__ inline int swz(int r) { return (r >> 1) & 7; }
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every extent: loads 0

enum Epi { kStore = 0, kAdd = 1, kSwiglu = 2, kPartial = 3 };

struct GemmArgs {
    int M, N, K;      // out is M x N; swiglu: W has 2N rows
    const uint16_t *A;
    int lda;          // A row pitch (elements)
    const uint16_t *W;
    void *out;
    int ldo;          // out row pitch (elements)
    const float *R;   // residual (add)
    int ldr;
    float *part;      // split-K partials [splits][M][Nw]
    int Nw;           // W rows = partial columns (N, or 2N for swiglu)
    int ksplit;       // K per split, a multiple of kTK
    int splits;
    int tiles_m, tiles_n;
    int group_m;      // M tiles per group of the tile order
    // optional, add epilogue with a split K range: the reduce also writes RMSNorm of each new
    // out row with weight nw to nout (bf16 [M][N]) -- the next layer's normed input
    const float *nw;
    float neps;
    uint16_t *nout;
    // optional, store epilogue with a split K range: the reduce also writes, for the columns
    // below cD (the x half of [x | z]), u = SiLU(conv(x)) of this one new token from the conv
    // history c0 (bf16 [M][3][cD], oldest first), weights cw [cD][4] and bias cb (nullable)
    const float *cw, *cb;
    const uint16_t *c0;
    const int32_t *chead;  // nullable: c0 is a ring, entry k in slot (chead[row] + k) mod 3
    uint16_t *cu;
    int cD;
};

__device__ inline float silu_f(float v) { return v * hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

// Logical tile order.  The hardware deals consecutive workgroup ids to the 8 XCDs in turn;
// the remap gives each XCD a contiguous range of logical ids, and within it tiles run in
// groups of group_m M tiles x all N tiles, column by column, so the workgroups resident on
// one XCD at a time share a few A row blocks and W row blocks in that XCD's L2.
__device__ inline void tile_of(const GemmArgs &a, int &tm, int &tn, int &split)
{
    const int total = a.tiles_m * a.tiles_n * a.splits;
    const int b = blockIdx.x;
    const int q = total / 8, r = total % 8, x = b % 8;
    const int L = x * q + min(x, r) + b / 8;
    const int ntiles = a.tiles_m * a.tiles_n;
    split = L / ntiles;
    const int t = L % ntiles;
    const int gsz = a.group_m * a.tiles_n;
    const int g = t / gsz, first = g * a.group_m;
    const int gm = min(a.group_m, a.tiles_m - first);
    tm = first + (t % gsz) % gm;
    tn = (t % gsz) / gm;
}

// Epilogue of a TM x TN tile: lane holds rows 4 (l / 16) + e, column l % 16 of every
// 16 x 16 MFMA tile of its wave's 16 FM x 16 FN block.
template <int FM, int FN, int kOutCols, int kEpi>
__device__ inline void store_tile_out(const GemmArgs &a, const f32x4 (&acc)[FM][FN], int m0, int n0, int wm, int wn,
                                      int lane, int split)
{
    const int erow = m0 + wm * 16 * FM + 4 * (lane >> 4);
    const int ecol = lane & 15;
    if constexpr (kEpi == kSwiglu) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int p = 0; p < FN / 2; ++p) {
                const int col = n0 + (wn * FN / 2 + p) * 16 + ecol;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = erow + i * 16 + e;
                    if (row < a.M && col < a.N)
                        static_cast<uint16_t *>(a.out)[static_cast<size_t>(row) * a.ldo + col] = __builtin_bit_cast(
                            uint16_t, static_cast<__bf16>(acc[i][2 * p][e] * silu_f(acc[i][2 * p + 1][e])));
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = n0 + wn * 16 * FN + j * 16 + ecol;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = erow + i * 16 + e;
                    if constexpr (kEpi == kPartial) {
                        if (row < a.M && col < a.Nw)
                            a.part[(static_cast<size_t>(split) * a.M + row) * a.Nw + col] = acc[i][j][e];
                    } else {
                        if (row >= a.M || col >= a.N) continue;
                        const size_t o = static_cast<size_t>(row) * a.ldo + col;
                        if constexpr (kEpi == kStore) {
                            static_cast<uint16_t *>(a.out)[o] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[i][j][e]));
                        } else {
                            static_cast<float *>(a.out)[o] = a.R[static_cast<size_t>(row) * a.ldr + col] + acc[i][j][e];
                        }
                    }
                }
            }
    }
}

template <int WGM, int WGN, int FM, int FN, int kEpi>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(GemmArgs a)
{
    // WGM x WGN waves, each a 16 FM x 16 FN block of 16 x 16 MFMA tiles
    constexpr int NT = 64 * WGM * WGN;
    constexpr int TM = 16 * FM * WGM, TN = 16 * FN * WGN;
    constexpr int RP = NT / 8;                 // tile rows per loader pass (8 threads per row)
    constexpr int LA = TM / RP, LW = TN / RP;  // 16-byte vectors per thread per K tile
    __shared__ __attribute__((aligned(16))) uint16_t As[2][TM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][TN * kPitch];

    int tm, tn, split;
    tile_of(a, tm, tn, split);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / WGN, wn = w % WGN;
    const int m0 = tm * TM;
    // Output columns of this tile: TN of them, or TN / 2 for the fused SwiGLU (the W tile
    // then holds TN / 2 rows of W1 and the same TN / 2 rows of W2, in alternating
    // 16-row blocks, so a wave's MFMA tiles 2p and 2p + 1 hold the two factors of the
    // same outputs in the same lanes).
    constexpr int kOutCols = kEpi == kSwiglu ? TN / 2 : TN;
    const int n0 = tn * kOutCols;
    const int kbeg = split * a.ksplit;
    const int kend = min(a.K, kbeg + a.ksplit);
    const int nk = kend > kbeg ? (kend - kbeg + kTK - 1) / kTK : 0;

    // Global -> register loaders: thread t moves 16-byte chunk c = t % 8 of rows
    // t / 8 + RP j of the A tile (j < LA) and of the W tile (j < LW); the row offsets below
    // exclude the chunk, which enters through the K index of load_tile.
    const int c = tid & 7, r0 = tid >> 3;
    const int rows_a = min(TM, a.M - m0);
    const Rsrc ra = make_rsrc(a.A + static_cast<size_t>(m0) * a.lda,
                              rows_a > 0 ? static_cast<uint32_t>(((rows_a - 1) * a.lda + a.K) * 2) : 0u);
    Rsrc rw, rw2;
    if constexpr (kEpi == kSwiglu) {
        const int rows = max(0, min(kOutCols, a.N - n0));
        const uint32_t ext = rows > 0 ? static_cast<uint32_t>(((rows - 1) * a.K + a.K) * 2) : 0u;
        rw = make_rsrc(a.W + static_cast<size_t>(n0) * a.K, ext);
        rw2 = make_rsrc(a.W + static_cast<size_t>(a.N + n0) * a.K, ext);
    } else {
        const int rows = max(0, min(TN, a.Nw - n0));
        rw = make_rsrc(a.W + static_cast<size_t>(n0) * a.K, rows > 0 ? static_cast<uint32_t>(rows * a.K * 2) : 0u);
        rw2 = rw;
    }
    uint32_t aoff[LA], woff[LW];
    bool wsecond[LW];
#pragma unroll
    for (int j = 0; j < LA; ++j) aoff[j] = static_cast<uint32_t>((r0 + RP * j) * a.lda * 2);
#pragma unroll
    for (int j = 0; j < LW; ++j) {
        const int r = r0 + RP * j;
        int wrow = r;
        wsecond[j] = false;
        if constexpr (kEpi == kSwiglu) {
            const int blk = r >> 4;
            wsecond[j] = (blk & 1) != 0;
            wrow = (blk >> 1) * 16 + (r & 15);
        }
        woff[j] = static_cast<uint32_t>(wrow * a.K * 2);
    }

    uint4 ra_v[LA], rw_v[LW];
    auto load_tile = [&](int kt) {
        const int k = kbeg + kt * kTK + c * 8;
        const bool in = k < kend;
        const uint32_t kb = static_cast<uint32_t>(k) * 2u;
#pragma unroll
        for (int j = 0; j < LA; ++j) ra_v[j] = buf_ld128(ra, in ? aoff[j] + kb : kOob);
#pragma unroll
        for (int j = 0; j < LW; ++j) rw_v[j] = buf_ld128(wsecond[j] ? rw2 : rw, in ? woff[j] + kb : kOob);
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int j = 0; j < LA; ++j)
            *reinterpret_cast<uint4 *>(&As[buf][(r0 + RP * j) * kPitch + ((c ^ swz(r0)) << 3)]) = ra_v[j];
#pragma unroll
        for (int j = 0; j < LW; ++j)
            *reinterpret_cast<uint4 *>(&Bs[buf][(r0 + RP * j) * kPitch + ((c ^ swz(r0)) << 3)]) = rw_v[j];
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Per K tile: the next tile's global loads are issued first and stay in flight while
    // the two 32-wide MFMA steps run on this tile's LDS buffer; then they are written to the
    // other buffer and one barrier ends the tile.  (Interleaving the LDS reads and writes with
    // the MFMAs through scheduling group barriers measured slower on 128 x 128 tiles, and
    // 256 x 256 tiles have no registers left for a second fragment set.)
    const int frow = lane & 15, fk = 8 * (lane >> 4);
    if (nk > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tile(kt + 1);
        // rows 16 m + frow: the swizzle depends on frow only (RP and 16 are multiples of 16)
        const uint16_t *as = &As[buf][(wm * 16 * FM + frow) * kPitch];
        const uint16_t *bs = &Bs[buf][(wn * 16 * FN + frow) * kPitch];
#pragma unroll
        for (int ks = 0; ks < kTK / 32; ++ks) {
            bf16x8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(as + i * 16 * kPitch + (((ks * 4 + (fk >> 3)) ^ swz(frow)) << 3));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const bf16x8 *>(bs + j * 16 * kPitch + (((ks * 4 + (fk >> 3)) ^ swz(frow)) << 3));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tile(buf ^ 1);
        __syncthreads();
    }

    store_tile_out<FM, FN, kOutCols, kEpi>(a, acc, m0, n0, wm, wn, lane, split);
}

// The same tile product with the operands loaded straight into LDS (buffer_load_dwordx4 ...
// lds: no register staging and no LDS-store phase in the instruction stream) through a ring
// of S stages, S - 1 of them in flight while one is multiplied.  A load-to-LDS instruction
// writes 64 lanes x 16 bytes contiguously (lane l at byte 16 l), i.e. 8 rows of a tile; lane l
// fetches the global chunk that the swizzle puts at its position, so the LDS layout is the
// one the fragment reads of gemm_kernel expect.  Lanes past a resource's extent (rows past M
// or N, K past the split) write zeros.  Used for 256 x 256 tiles on 8 waves with S = 2 (128 KB,
// one stage in flight while one is multiplied, as in gemm_kernel): measured 9-16 % faster than
// register staging on the 1.7B prefill projections.  For 128 x 128 tiles a 4-stage ring (one
// workgroup per CU, three stages in flight) measured slower than two register-staged
// workgroups per CU, on prefill and decode shapes alike.
template <int WGM, int WGN, int FM, int FN, int kEpi, int S>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_ring_kernel(GemmArgs a)
{
    constexpr int NW = WGM * WGN;
    constexpr int TM = 16 * FM * WGM, TN = 16 * FN * WGN;
    constexpr int kRowsPerLd = 8;                                // rows of one load-to-LDS instruction
    constexpr int kLdPerWave = (TM + TN) / (kRowsPerLd * NW);    // per wave and stage
    static_assert((TM + TN) % (kRowsPerLd * NW) == 0 && TM % (kRowsPerLd * kLdPerWave) == 0,
                  "every load instruction of a wave must fall in one operand");
    static_assert(S >= 2 && S <= 4, "the stage waits below cover at most two stages in flight after the current one");
    // SwiGLU tiles alternate 16-row blocks of W1 and W2 rows; with these the block of the
    // wave's instruction j is W2 exactly when bit 1 of j is set (a compile-time choice)
    static_assert(kLdPerWave % 4 == 0 && (TM / kRowsPerLd) % 4 == 0, "W1 / W2 block parity must follow j");
    constexpr int kStageElems = (TM + TN) * kPitch;
    __shared__ __attribute__((aligned(16))) uint16_t ring[S][kStageElems];

    int tm, tn, split;
    tile_of(a, tm, tn, split);
    // the wave index in a scalar register: the operand, resource and LDS destination of every
    // load instruction derive from it, and must be wave-uniform
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w / WGN, wn = w % WGN;
    const int m0 = tm * TM;
    constexpr int kOutCols = kEpi == kSwiglu ? TN / 2 : TN;
    const int n0 = tn * kOutCols;
    const int kbeg = split * a.ksplit;
    const int kend = min(a.K, kbeg + a.ksplit);
    const int nk = kend > kbeg ? (kend - kbeg + kTK - 1) / kTK : 0;

    const int rows_a = min(TM, a.M - m0);
    const Rsrc ra = make_rsrc(a.A + static_cast<size_t>(m0) * a.lda,
                              rows_a > 0 ? static_cast<uint32_t>(((rows_a - 1) * a.lda + a.K) * 2) : 0u);
    Rsrc rw, rw2;
    if constexpr (kEpi == kSwiglu) {
        const int rows = max(0, min(kOutCols, a.N - n0));
        const uint32_t ext = static_cast<uint32_t>(rows * a.K * 2);
        rw = make_rsrc(a.W + static_cast<size_t>(n0) * a.K, ext);
        rw2 = make_rsrc(a.W + static_cast<size_t>(a.N + n0) * a.K, ext);
    } else {
        const int rows = max(0, min(TN, a.Nw - n0));
        rw = make_rsrc(a.W + static_cast<size_t>(n0) * a.K, static_cast<uint32_t>(rows * a.K * 2));
        rw2 = rw;
    }

    // The wave's load instructions: instruction j covers rows 8 g .. 8 g + 7 of the stage
    // (A rows first, then W rows), g = w kLdPerWave + j; lane l loads row 8 g + l / 8 at the
    // chunk that the swizzle stores at position l % 8.
    const bool is_a = w * kLdPerWave * kRowsPerLd < TM;          // wave-uniform
    uint32_t off[kLdPerWave];
    int qk[kLdPerWave];                                          // the lane's K offset in a stage
#pragma unroll
    for (int j = 0; j < kLdPerWave; ++j) {
        const int g = w * kLdPerWave + j;
        const int gop = is_a ? g : g - TM / kRowsPerLd;            // instruction within its operand
        const int r = gop * kRowsPerLd + (lane >> 3);              // row in its operand tile
        const int q = (lane & 7) ^ swz(r);
        qk[j] = q * 8;
        if (is_a) {
            off[j] = static_cast<uint32_t>(r * a.lda * 2);
        } else {
            int wrow = r;
            if constexpr (kEpi == kSwiglu) wrow = ((r >> 4) >> 1) * 16 + (r & 15);
            off[j] = static_cast<uint32_t>(wrow * a.K * 2);
        }
    }
    auto issue = [&](int kt, int slot) {
#pragma unroll
        for (int j = 0; j < kLdPerWave; ++j) {
            const int k = kbeg + kt * kTK + qk[j];
            const uint32_t o = k < kend ? off[j] + static_cast<uint32_t>(k) * 2u : kOob;
            uint16_t *dst = &ring[slot][(w * kLdPerWave + j) * kRowsPerLd * kPitch];
            const Rsrc rs = is_a ? ra : ((kEpi == kSwiglu && ((j >> 1) & 1)) ? rw2 : rw);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)dst,
                                                     16, o, 0, 0, 0);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15, fk = 8 * (lane >> 4);
#pragma unroll
    for (int p = 0; p < S - 1; ++p)
        if (p < nk) issue(p, p);
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt has landed for this wave once only the stages issued after it are
        // outstanding; the barrier then covers every wave's loads of it, and every wave has
        // finished reading the slot that the next issue overwrites (stage kt - 1's).
        const int after = min(S - 2, nk - 1 - kt);
        if (after >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLdPerWave));
        else if (after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLdPerWave));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        barrier_no_fence();
        if (kt + S - 1 < nk) issue(kt + S - 1, (kt + S - 1) % S);
        const uint16_t *st = ring[kt % S];
        const uint16_t *as = st + (wm * 16 * FM + frow) * kPitch;
        const uint16_t *bs = st + (TM + wn * 16 * FN + frow) * kPitch;
#pragma unroll
        for (int ks = 0; ks < kTK / 32; ++ks) {
            bf16x8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(as + i * 16 * kPitch + (((ks * 4 + (fk >> 3)) ^ swz(frow)) << 3));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const bf16x8 *>(bs + j * 16 * kPitch + (((ks * 4 + (fk >> 3)) ^ swz(frow)) << 3));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
    store_tile_out<FM, FN, kOutCols, kEpi>(a, acc, m0, n0, wm, wn, lane, split);
}

// Skinny products: the decode step's projections, a few hundred token rows against 2K-16K
// weight rows.  Every weight is used by few rows, so the work is streaming operands (the
// weights once from memory, the token rows again for every column tile from L2), and the
// kernel is built for loads in flight and for independent waves:
// - the K range of a tile is split over the workgroup's KW waves (contiguous 64-wide
//   blocks per wave), and each wave streams its own blocks through its own NS LDS slots
//   with loads straight into LDS (buffer_load_dwordx4 ... lds: 8 rows x 128 bytes per
//   instruction, whole cache lines), NS - 1 blocks in flight while the current one is
//   multiplied; a wave reads only what it loaded itself, so the loop has no barrier;
// - fragments are read from LDS with the XOR swizzle of the other kernels (conflict-free);
// - at the end the waves' fp32 tiles are summed through LDS in wave order (a fixed order:
//   the result does not depend on timing), so a tile needs no partial sums in memory
//   unless its K range is also split across workgroups (a.splits > 1: kPartial, summed by
//   the reduce kernels below).
// Rows past M and W rows past the tile's extent load zeros through the buffer resources; K
// past the wave's range loads zeros through kOob.  The epilogue (bf16 store with the optional
// conv of the new token, fp32 residual add, SwiGLU or fp32 partials) reads the summed tile
// in row order, 4 consecutive outputs per thread, so its global traffic is whole vectors.
template <int FM, int FN, int NS, int kEpi>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs a)
{
    constexpr int KW = 4;
    constexpr int TM = 16 * FM, TN = 16 * FN;
    constexpr int kOutCols = kEpi == kSwiglu ? TN / 2 : TN;
    constexpr int kRows = TM + TN;                 // rows of one block: A rows, then W rows
    constexpr int kLd = kRows / 8;                 // load instructions per block
    constexpr int kSlot = kRows * kPitch;          // elements of one slot
    static_assert(kEpi != kSwiglu || FN % 2 == 0, "SwiGLU tiles pair W1 and W2 blocks");
    static_assert(FM * FN * 64 * 16 <= NS * kSlot * 2, "the summing area of a wave fits in its slots");
    static_assert(NS >= 2 && (NS - 1) * kLd <= 63, "the wait count of NS - 1 blocks in flight must fit vmcnt");
    __shared__ __attribute__((aligned(16))) uint16_t lds[KW][NS][kSlot];

    int tm, tn, split;
    tile_of(a, tm, tn, split);
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m0 = tm * TM, n0 = tn * kOutCols;
    const int kbeg = split * a.ksplit;
    const int kend = min(a.K, kbeg + a.ksplit);
    const int nb = kend > kbeg ? (kend - kbeg + kTK - 1) / kTK : 0;
    const int b0 = nb * w / KW, b1 = nb * (w + 1) / KW;

    const int rows_a = min(TM, a.M - m0);
    const Rsrc ra = make_rsrc(a.A + static_cast<size_t>(m0) * a.lda,
                              rows_a > 0 ? static_cast<uint32_t>(((rows_a - 1) * a.lda + a.K) * 2) : 0u);
    Rsrc rw, rw2;
    if constexpr (kEpi == kSwiglu) {
        const int rows = max(0, min(kOutCols, a.N - n0));
        const uint32_t ext = static_cast<uint32_t>(rows * a.K * 2);
        rw = make_rsrc(a.W + static_cast<size_t>(n0) * a.K, ext);
        rw2 = make_rsrc(a.W + static_cast<size_t>(a.N + n0) * a.K, ext);
    } else {
        const int rows = max(0, min(TN, a.Nw - n0));
        rw = make_rsrc(a.W + static_cast<size_t>(n0) * a.K, static_cast<uint32_t>(rows * a.K * 2));
        rw2 = rw;
    }
    // Load instruction j of a block covers slot rows 8 j .. 8 j + 7; lane l loads row
    // 8 j + l / 8 at the 16-byte chunk that the swizzle stores at position l % 8.
    uint32_t off[kLd];
    int qk[kLd];
#pragma unroll
    for (int j = 0; j < kLd; ++j) {
        const int r = 8 * j + (lane >> 3);
        qk[j] = ((lane & 7) ^ swz(r)) * 8;
        if (8 * j < TM) {
            off[j] = static_cast<uint32_t>(r * a.lda * 2);
        } else {
            const int wr = r - TM;
            // SwiGLU: W rows alternate 16-row blocks of W1 and W2 (the W2 resource)
            const int wrow = kEpi == kSwiglu ? ((wr >> 4) >> 1) * 16 + (wr & 15) : wr;
            off[j] = static_cast<uint32_t>(wrow * a.K * 2);
        }
    }
    auto issue = [&](int b, int slot) {
        // blocks past the wave's range: every K index is past the limit
        const int lim = __builtin_amdgcn_readfirstlane(b < b1 ? kend : INT32_MIN);
        const int kb = kbeg + b * kTK;
#pragma unroll
        for (int j = 0; j < kLd; ++j) {
            const int k = kb + qk[j];
            const uint32_t o = k < lim ? off[j] + static_cast<uint32_t>(k) * 2u : kOob;
            const bool w2 = kEpi == kSwiglu && 8 * j >= TM && (((8 * j - TM) >> 4) & 1);
            const Rsrc rs = 8 * j < TM ? ra : (w2 ? rw2 : rw);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void *)&lds[w][slot][8 * j * kPitch], 16, o, 0, 0, 0);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int frow = lane & 15, fk = 8 * (lane >> 4);
    auto mult = [&](int slot) {
        const uint16_t *as = &lds[w][slot][frow * kPitch];
        const uint16_t *bs = &lds[w][slot][(TM + frow) * kPitch];
        bf16x8 af[2][FM], bf[2][FN];
#pragma unroll
        for (int h = 0; h < kTK / 32; ++h) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[h][i] = *reinterpret_cast<const bf16x8 *>(as + i * 16 * kPitch + (((h * 4 + (fk >> 3)) ^ swz(frow)) << 3));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[h][j] = *reinterpret_cast<const bf16x8 *>(bs + j * 16 * kPitch + (((h * 4 + (fk >> 3)) ^ swz(frow)) << 3));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int h = 0; h < kTK / 32; ++h)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[h][i], bf[h][j], acc[i][j], 0, 0, 0);
    };

    // Blocks b + 1 .. b + NS - 1 are in flight while block b is multiplied; every iteration
    // issues the same loads (blocks past the range load zeros), so one wait count fits every
    // path.  A slot is overwritten only after the products that read it: their LDS reads
    // completed before the MFMAs that consume them.
    // The epilogue's thread map: thread t owns 4 consecutive output columns of a row, so
    // global reads and writes are whole 8- or 16-byte vectors along rows.
    constexpr int kTpr = kOutCols / 4;            // threads per output row
    constexpr int kRpp = 256 / kTpr;              // rows per pass
    constexpr int kPasses = (TM + kRpp - 1) / kRpp;
    static_assert(kOutCols % 4 == 0 && 256 % kTpr == 0, "epilogue thread map");
    const int tid = threadIdx.x;
    const int c4 = 4 * (tid % kTpr);              // first output column in the tile
    const int col = n0 + c4;
    const bool vec_out = kEpi == kPartial ? (a.Nw % 4 == 0 && (reinterpret_cast<uintptr_t>(a.part) & 15u) == 0) :
                         kEpi == kAdd ? (a.ldo % 4 == 0 && a.ldr % 4 == 0 &&
                                         (reinterpret_cast<uintptr_t>(a.out) & 15u) == 0 &&
                                         (reinterpret_cast<uintptr_t>(a.R) & 15u) == 0)
                                      : (a.ldo % 4 == 0 && (reinterpret_cast<uintptr_t>(a.out) & 7u) == 0);

    if (b0 < b1) {
#pragma unroll
        for (int q = 0; q < NS - 1; ++q) issue(b0 + q, q);
    }
    // The conv of the new token (store epilogue with a.cu): its inputs are loaded here, after
    // the first blocks' loads and before the K loop, so that their latency hides behind the
    // products instead of following them: the three ring slots of every row of the thread
    // (the ring head only selects among them), the heads, the weights and the bias of its 4
    // columns.  conv_fusable guarantees whole 4-column groups (vec_out) here.
    [[maybe_unused]] uint2 hs[kPasses][3];
    [[maybe_unused]] int hd[kPasses];
    [[maybe_unused]] float4 cwv[4];
    [[maybe_unused]] float cbs[4];
    const bool conv = kEpi == kStore && a.cu != nullptr && col < a.cD && vec_out;
    if constexpr (kEpi == kStore) {
        if (conv) {
#pragma unroll
            for (int pass = 0; pass < kPasses; ++pass) {
                const int r = pass * kRpp + tid / kTpr, row = m0 + r;
                const bool ok = r < TM && row < a.M;
                const uint16_t *h = a.c0 + static_cast<size_t>(ok ? row : 0) * 3 * a.cD + col;
#pragma unroll
                for (int k = 0; k < 3; ++k) hs[pass][k] = *reinterpret_cast<const uint2 *>(h + k * a.cD);
                hd[pass] = ok && a.chead != nullptr ? a.chead[row] : 0;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) cwv[u] = *reinterpret_cast<const float4 *>(a.cw + static_cast<size_t>(col + u) * 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) cbs[u] = a.cb != nullptr ? a.cb[col + u] : 0.0f;
        }
    }
    if (b0 < b1) {
        int slot = 0;
        for (int b = b0; b < b1; ++b) {
            issue(b + NS - 1, slot == 0 ? NS - 1 : slot - 1);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * kLd));
            asm volatile("" ::: "memory");
            mult(slot);
            __builtin_amdgcn_sched_barrier(0);
            slot = slot == NS - 1 ? 0 : slot + 1;
        }
        // the last issues (zeros) may still be writing their slots
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }

    // the waves' tiles summed in wave order, each wave's tile in its own slots
    f32x4 *red = reinterpret_cast<f32x4 *>(&lds[w][0][0]);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) red[(i * FN + j) * 64 + lane] = acc[i][j];
    __syncthreads();

    // Epilogue in row order (thread map above): element (r, c) of the product tile (i, j)
    // sits in lane c % 16 + 16 ((r % 16) / 4), component r % 4.
    const int cblk = c4 >> 4, clane = c4 & 15;
    auto summed = [&](int tile, int ln, int e) {
        const float *base = reinterpret_cast<const float *>(&lds[0][0][0]);
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < KW; ++q)
            v += base[q * (NS * kSlot / 2) + ((tile * 64 + ln) * 4 + e)];
        return v;
    };
    uint2 xpk[kPasses];                           // the stored x of each pass (conv input)
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
        const int r = pass * kRpp + tid / kTpr;   // row in the tile
        const int row = m0 + r;
        if (r >= TM || row >= a.M) continue;
        const int ln0 = clane + 16 * ((r & 15) >> 2), e = r & 3;
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if constexpr (kEpi == kSwiglu) {
                const int t1 = (r >> 4) * FN + 2 * cblk;
                v[u] = summed(t1, ln0 + u, e) * silu_f(summed(t1 + 1, ln0 + u, e));
            } else {
                v[u] = summed((r >> 4) * FN + cblk, ln0 + u, e);
            }
        }
        const int ncols = kEpi == kPartial ? a.Nw : a.N;
        if constexpr (kEpi == kPartial) {
            float *dst = a.part + (static_cast<size_t>(split) * a.M + row) * a.Nw + col;
            if (vec_out && col + 3 < ncols) {
                *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (col + u < ncols) dst[u] = v[u];
            }
        } else if constexpr (kEpi == kAdd) {
            float *dst = static_cast<float *>(a.out) + static_cast<size_t>(row) * a.ldo + col;
            const float *res = a.R + static_cast<size_t>(row) * a.ldr + col;
            if (vec_out && col + 3 < ncols) {
                const float4 rv = *reinterpret_cast<const float4 *>(res);
                *reinterpret_cast<float4 *>(dst) = make_float4(rv.x + v[0], rv.y + v[1], rv.z + v[2], rv.w + v[3]);
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (col + u < ncols) dst[u] = res[u] + v[u];
            }
        } else {
            uint16_t *dst = static_cast<uint16_t *>(a.out) + static_cast<size_t>(row) * a.ldo + col;
            if (vec_out && col + 3 < ncols) {
                const uint2 pk = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
                *reinterpret_cast<uint2 *>(dst) = pk;
                if constexpr (kEpi == kStore) xpk[pass] = pk;
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (col + u < ncols) dst[u] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[u]));
            }
        }
    }
    if constexpr (kEpi == kStore) {
        // the conv of the one new token for the columns below cD, in the order and precision
        // of conv_silu_kernel: x as stored (bf16), the history as stored
        if (conv) {
#pragma unroll
            for (int pass = 0; pass < kPasses; ++pass) {
                const int r = pass * kRpp + tid / kTpr, row = m0 + r;
                if (r >= TM || row >= a.M) continue;
                const uint2 pk = xpk[pass];
                const float xs[4] = {bf16lo(pk.x), bf16hi(pk.x), bf16lo(pk.y), bf16hi(pk.y)};
                const int s0 = ring_slot(hd[pass], 0);
                // selected word by word: a select between whole uint2 values becomes a select
                // between their addresses, which puts the array in scratch memory
                const uint2 a0 = hs[pass][0], a1 = hs[pass][1], a2 = hs[pass][2];
                auto pick = [s0](uint32_t v0, uint32_t v1, uint32_t v2) { return s0 == 0 ? v0 : (s0 == 1 ? v1 : v2); };
                const uint2 h0 = make_uint2(pick(a0.x, a1.x, a2.x), pick(a0.y, a1.y, a2.y));
                const uint2 h1 = make_uint2(pick(a1.x, a2.x, a0.x), pick(a1.y, a2.y, a0.y));
                const uint2 h2 = make_uint2(pick(a2.x, a0.x, a1.x), pick(a2.y, a0.y, a1.y));
                const float w0[4] = {bf16lo(h0.x), bf16hi(h0.x), bf16lo(h0.y), bf16hi(h0.y)};
                const float w1[4] = {bf16lo(h1.x), bf16hi(h1.x), bf16lo(h1.y), bf16hi(h1.y)};
                const float w2[4] = {bf16lo(h2.x), bf16hi(h2.x), bf16lo(h2.y), bf16hi(h2.y)};
                float uu[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float pre = __builtin_fmaf(cwv[u].x, w0[u], cbs[u]);
                    pre = __builtin_fmaf(cwv[u].y, w1[u], pre);
                    pre = __builtin_fmaf(cwv[u].z, w2[u], pre);
                    pre = __builtin_fmaf(cwv[u].w, xs[u], pre);
                    uu[u] = silu_f(pre);
                }
                *reinterpret_cast<uint2 *>(a.cu + static_cast<size_t>(row) * a.cD + col) =
                    make_uint2(pack_bf16(uu[0], uu[1]), pack_bf16(uu[2], uu[3]));
            }
        }
    }
}

// Sums the split partials in split order and applies the epilogue; one thread per kVec
// consecutive outputs of a row (kVec = 4: 16-byte partial loads, when N, the row pitches and
// the output are aligned for them; see vec_ok).
template <int kEpi, int kVec>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs a)
{
    const int nvec = a.N / kVec;
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= static_cast<size_t>(a.M) * nvec) return;
    const int row = static_cast<int>(i / nvec), col = static_cast<int>(i % nvec) * kVec;
    const size_t stride = static_cast<size_t>(a.M) * a.Nw;
    const float *p = a.part + static_cast<size_t>(row) * a.Nw + col;
    float s[kVec] = {}, g[kVec] = {};
    for (int k = 0; k < a.splits; ++k) {
        if constexpr (kVec == 4) {
            const float4 v = *reinterpret_cast<const float4 *>(p + k * stride);
            s[0] += v.x, s[1] += v.y, s[2] += v.z, s[3] += v.w;
            if constexpr (kEpi == kSwiglu) {
                const float4 w = *reinterpret_cast<const float4 *>(p + k * stride + a.N);
                g[0] += w.x, g[1] += w.y, g[2] += w.z, g[3] += w.w;
            }
        } else {
            s[0] += p[k * stride];
            if constexpr (kEpi == kSwiglu) g[0] += p[k * stride + a.N];
        }
    }
    const size_t o = static_cast<size_t>(row) * a.ldo + col;
    if constexpr (kEpi == kAdd) {
        const float *r = a.R + static_cast<size_t>(row) * a.ldr + col;
        if constexpr (kVec == 4) {
            const float4 rv = *reinterpret_cast<const float4 *>(r);
            *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + o) =
                make_float4(rv.x + s[0], rv.y + s[1], rv.z + s[2], rv.w + s[3]);
        } else {
            static_cast<float *>(a.out)[o] = r[0] + s[0];
        }
    } else {
        float v[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) v[e] = kEpi == kSwiglu ? s[e] * silu_f(g[e]) : s[e];
        uint16_t *dst = static_cast<uint16_t *>(a.out) + o;
        if constexpr (kVec == 4) {
            const uint2 pk = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
            *reinterpret_cast<uint2 *>(dst) = pk;
            if constexpr (kEpi == kStore) {
                if (a.cu != nullptr && col < a.cD) {
                    // the conv of the one new token, in the order and precision of
                    // conv_silu_kernel: x as stored (bf16), the history as stored
                    const float xs[4] = {bf16lo(pk.x), bf16hi(pk.x), bf16lo(pk.y), bf16hi(pk.y)};
                    const uint16_t *h = a.c0 + static_cast<size_t>(row) * 3 * a.cD + col;
                    const int hd = a.chead != nullptr ? a.chead[row] : 0;
                    const uint2 h0 = *reinterpret_cast<const uint2 *>(h + ring_slot(hd, 0) * a.cD);
                    const uint2 h1 = *reinterpret_cast<const uint2 *>(h + ring_slot(hd, 1) * a.cD);
                    const uint2 h2 = *reinterpret_cast<const uint2 *>(h + ring_slot(hd, 2) * a.cD);
                    const float w0[4] = {bf16lo(h0.x), bf16hi(h0.x), bf16lo(h0.y), bf16hi(h0.y)};
                    const float w1[4] = {bf16lo(h1.x), bf16hi(h1.x), bf16lo(h1.y), bf16hi(h1.y)};
                    const float w2[4] = {bf16lo(h2.x), bf16hi(h2.x), bf16lo(h2.y), bf16hi(h2.y)};
                    float u[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float4 cwv = *reinterpret_cast<const float4 *>(a.cw + static_cast<size_t>(col + e) * 4);
                        float pre = __builtin_fmaf(cwv.x, w0[e], a.cb ? a.cb[col + e] : 0.0f);
                        pre = __builtin_fmaf(cwv.y, w1[e], pre);
                        pre = __builtin_fmaf(cwv.z, w2[e], pre);
                        pre = __builtin_fmaf(cwv.w, xs[e], pre);
                        u[e] = silu_f(pre);
                    }
                    *reinterpret_cast<uint2 *>(a.cu + static_cast<size_t>(row) * a.cD + col) =
                        make_uint2(pack_bf16(u[0], u[1]), pack_bf16(u[2], u[3]));
                }
            }
        } else {
            dst[0] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[0]));
        }
    }
}

// Whether the reduce may move 4 outputs per thread: N and the row pitches multiples of 4,
// the output 8-byte (bf16) or 16-byte (fp32) aligned, the residual 16-byte aligned.
inline bool vec_ok(const GemmArgs &a, int epi)
{
    const uintptr_t o = reinterpret_cast<uintptr_t>(a.out);
    if (a.N % 4 || a.ldo % 4) return false;
    if (epi == kAdd) return (o & 15u) == 0 && a.ldr % 4 == 0 && (reinterpret_cast<uintptr_t>(a.R) & 15u) == 0;
    return (o & 7u) == 0;
}

// The reduce of a split add epilogue fused with the RMSNorm that follows it: one workgroup
// per row; thread t sums, for elements 8 (256 c + t) .. + 7 (c < NCH), the splits in split
// order and adds the residual -- the arithmetic of gemm_reduce_kernel<kAdd, 4> -- writes the
// new row, then normalises it with the arithmetic of the 16-byte RMSNorm (sum of squares per
// thread in element order, then across the wave and the 4 waves), so that the result is
// bitwise that of the two kernels run one after the other.  N % 8 == 0, N <= 2048 NCH,
// ldo == ldr == N, out, R, nw and nout 16-byte aligned.
template <int NCH>
__global__ __launch_bounds__(256) void gemm_reduce_add_norm_kernel(GemmArgs a)
{
    const int r = blockIdx.x;
    if (r >= a.M) return;
    const int d = a.N;
    const size_t stride = static_cast<size_t>(a.M) * a.Nw;
    const float *prow = a.part + static_cast<size_t>(r) * a.Nw;
    float *orow = static_cast<float *>(a.out) + static_cast<size_t>(r) * d;
    const float *rrow = a.R + static_cast<size_t>(r) * d;
    float v[NCH][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int i = (c * 256 + threadIdx.x) * 8;
        if (i < d) {
            float acc[8] = {};
            for (int k = 0; k < a.splits; ++k) {
                const float4 p0 = *reinterpret_cast<const float4 *>(prow + k * stride + i);
                const float4 p1 = *reinterpret_cast<const float4 *>(prow + k * stride + i + 4);
                acc[0] += p0.x, acc[1] += p0.y, acc[2] += p0.z, acc[3] += p0.w;
                acc[4] += p1.x, acc[5] += p1.y, acc[6] += p1.z, acc[7] += p1.w;
            }
            const float4 r0 = *reinterpret_cast<const float4 *>(rrow + i);
            const float4 r1 = *reinterpret_cast<const float4 *>(rrow + i + 4);
            const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) v[c][e] = rv[e] + acc[e];
            *reinterpret_cast<float4 *>(orow + i) = make_float4(v[c][0], v[c][1], v[c][2], v[c][3]);
            *reinterpret_cast<float4 *>(orow + i + 4) = make_float4(v[c][4], v[c][5], v[c][6], v[c][7]);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[c][e], v[c][e], ss);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = __builtin_amdgcn_rsqf(tot / static_cast<float>(d) + a.neps);
    uint16_t *nrow = a.nout + static_cast<size_t>(r) * d;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int i = (c * 256 + threadIdx.x) * 8;
        if (i < d) {
            const float4 w0 = *reinterpret_cast<const float4 *>(a.nw + i);
            const float4 w1 = *reinterpret_cast<const float4 *>(a.nw + i + 4);
            const float ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pk[e] = pack_bf16(v[c][2 * e] * inv * ws[2 * e], v[c][2 * e + 1] * inv * ws[2 * e + 1]);
            *reinterpret_cast<uint4 *>(nrow + i) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
    }
}

// ---------------------------------------------------------------- host side
struct Plan {
    int fm, fn;       // tile config
    bool w8;          // 256 x 256 tiles on 8 waves (4 along M x 2 along N), gemm_ring_kernel
    bool stream;      // gemm_stream_kernel with a 16 fm x 16 fn tile and ns LDS slots per wave
    int ns;
    int ring;         // > 0: 128 x 128 tiles on gemm_ring_kernel with this many stages
    int splits, ksplit;
    int tiles_m, tiles_n;
    size_t part_bytes;
};

// The stream kernel's tile shapes (FM, FN, LDS slots per wave).  Two slots measured best
// (three to five slots per wave, i.e. more blocks in flight, were slower on every decode
// shape: the operand traffic through L2, not the latency, bounds these products).
constexpr int kStreamShapes[][3] = {{4, 4, 2}, {4, 2, 2}, {2, 4, 2}, {2, 2, 2}};

// Plan of a skinny product: the stream kernel's shape and split count of least estimated
// time, or, for SwiGLU, 128 x 128 tiles on the two-stage ring kernel.  SAMBA_GEMM_STREAM =
// "FMxFNnNSsS" (the n and s parts optional) forces a built stream shape, "rNSsS" the ring
// kernel with NS stages, for tests and timing.
inline bool plan_stream(int M, int N, int K, int epi, Plan &p)
{
    const int Nw = epi == kSwiglu ? 2 * N : N;
    const int nk = (K + kTK - 1) / kTK;
    auto grid_of = [&](int fm, int fn, int s) {
        const int TM = 16 * fm, TN = 16 * fn;
        const long long tn = s > 1 || epi != kSwiglu ? (Nw + TN - 1) / TN : (N + TN / 2 - 1) / (TN / 2);
        return static_cast<long long>((M + TM - 1) / TM) * tn * s;
    };
    int fm = 0, fn = 0, ns = 0, s = 1;
    const char *force = getenv("SAMBA_GEMM_STREAM");
    int st = 0;
    if (force != nullptr && force[0] == 'r') {
        if (sscanf(force, "r%ds%d", &st, &s) < 1 || st < 2 || st > 4 || s < 1) return false;
    } else if ((force == nullptr || force[0] == '\0') && epi == kSwiglu &&
               static_cast<long long>((M + 127) / 128) * ((N + 63) / 64) >= 128) {
        // SwiGLU: the W1 / W2 pairs double the weight rows per output, and 128 x 128 tiles
        // on the two-stage ring, two workgroups per CU, measured faster than the stream
        // kernel (36 vs 52 us on the 1.7B MLP at 256 rows)
        st = 2;
    }
    if (st > 0) {
        p.stream = false;
        p.w8 = false;
        p.ring = st;
        p.fm = 4;
        p.fn = 4;
        const int kt_per = (nk + s - 1) / s;
        p.ksplit = std::max(1, kt_per) * kTK;
        p.splits = nk > 0 ? (nk + kt_per - 1) / kt_per : 1;
        p.tiles_m = (M + 127) / 128;
        p.tiles_n = p.splits > 1 || epi != kSwiglu ? (Nw + 127) / 128 : (N + 63) / 64;
        p.part_bytes = p.splits > 1 ? static_cast<size_t>(p.splits) * M * Nw * sizeof(float) : 0;
        return true;
    }
    if (force != nullptr && force[0] != '\0') {
        const char *q = force;
        char *e = nullptr;
        fm = static_cast<int>(strtol(q, &e, 10));
        if (e == q || *e != 'x') return false;
        q = e + 1;
        fn = static_cast<int>(strtol(q, &e, 10));
        if (e == q) return false;
        q = e;
        if (*q == 'n') {
            ns = static_cast<int>(strtol(q + 1, &e, 10));
            q = e;
        }
        if (*q == 's') {
            s = static_cast<int>(strtol(q + 1, &e, 10));
            q = e;
        }
        if (*q != '\0' || s < 1 || (epi == kSwiglu && fn % 2 != 0)) return false;
        bool known = false;
        for (const auto &sh : kStreamShapes)
            if (sh[0] == fm && sh[1] == fn && (ns == 0 || sh[2] == ns)) {
                known = true;
                ns = sh[2];
                break;
            }
        if (!known) return false;
    } else {
        // Estimated time (microseconds) of each shape and split count, fitted to the decode
        // projections measured on MI355X: a workgroup streams its operand bytes at about
        // 55 GB/s when 128 or more run (up to twice that when few do), the chip at most
        // about 11 TB/s; plus ~4 us of latency and ~4 us for the reduce of a split K range.
        double best = 1e30;
        for (const auto &sh : kStreamShapes) {
            if (epi == kSwiglu && sh[1] % 2 != 0) continue;
            const int lds = 4 * sh[2] * 16 * (sh[0] + sh[1]) * 128;
            const int per_cu = std::max(1, (160 << 10) / lds);
            for (int ss = 1; ss <= 8; ss *= 2) {
                if (ss > 1 && nk < 4 * ss) break;
                const long long g = grid_of(sh[0], sh[1], ss);
                const double kslice = static_cast<double>((nk + ss - 1) / ss) * kTK;
                const double wg_bytes = kslice * 16.0 * (sh[0] + sh[1]) * 2.0;
                const double total = wg_bytes * static_cast<double>(g);
                const double rounds = std::ceil(static_cast<double>(g) / (256.0 * per_cu));
                const double cu_rate = 55e9 * std::min(2.0, std::max(1.0, 128.0 / static_cast<double>(g)));
                const double t = 4.0 + std::max(total / 11e12, rounds * wg_bytes / cu_rate) * 1e6 + (ss > 1 ? 4.0 : 0.0);
                if (t < best) {
                    best = t;
                    fm = sh[0], fn = sh[1], ns = sh[2], s = ss;
                }
            }
        }
        if (fm == 0) return false;
    }
    p.stream = true;
    p.w8 = false;
    p.fm = fm;
    p.fn = fn;
    p.ns = ns;
    const int kt_per = (nk + s - 1) / s;
    p.ksplit = std::max(1, kt_per) * kTK;
    p.splits = nk > 0 ? (nk + kt_per - 1) / kt_per : 1;
    const int TM = 16 * fm, TN = 16 * fn;
    p.tiles_m = (M + TM - 1) / TM;
    p.tiles_n = p.splits > 1 || epi != kSwiglu ? (Nw + TN - 1) / TN : (N + TN / 2 - 1) / (TN / 2);
    p.part_bytes = p.splits > 1 ? static_cast<size_t>(p.splits) * M * Nw * sizeof(float) : 0;
    return true;
}

// Tile shape and split count for a problem.  Large problems take 256 x 256 tiles (one
// 8-wave workgroup per CU, 128 KB of LDS); problems with fewer than 256 such tiles take
// 128 x 128 tiles (two per CU), and if there are fewer than 256 of those, the K range is
// split (each split keeps at least 4 K tiles) until about 256 workgroups exist.  Measured on
// the decode step's projections (256 rows): aiming at 512 workgroups instead doubles the
// fp32 partial bytes (each split writes as many as the weights it reads) and made the step
// 3 % slower; 1024, 6-12 % slower.
inline Plan plan(int M, int N, int K, int epi)
{
    Plan p{};
    const int Nw = epi == kSwiglu ? 2 * N : N;
    {
        // skinny products (the decode step) stream the weights; 32-bit buffer offsets bound
        // the operand sizes it takes
        const char *off = getenv("SAMBA_GEMM_STREAM");
        const bool no_stream = off != nullptr && strcmp(off, "0") == 0;
        if (!no_stream && M <= 256 && static_cast<long long>(M) * K * 2 < (1ll << 31) &&
            static_cast<long long>(Nw) * K * 2 < (1ll << 31) && plan_stream(M, N, K, epi, p))
            return p;
    }
    auto tiles = [&](int tm, int tn) {
        const long long outc = epi == kSwiglu ? tn / 2 : tn;
        return static_cast<long long>((M + tm - 1) / tm) * ((N + outc - 1) / outc);
    };
    const char *force = getenv("SAMBA_GEMM_TILE");  // "128" / "256": tile choice for tests and timing
    const bool f128 = force != nullptr && strcmp(force, "128") == 0;
    const bool f256 = force != nullptr && strcmp(force, "256") == 0;
    if (f256 || (!f128 && tiles(256, 256) >= 256)) {
        p.fm = 8;
        p.fn = 8;
        p.w8 = true;
    } else {
        p.fm = 4;
        p.fn = 4;
    }
    const int TM = 32 * p.fm, TN = 32 * p.fn;
    const int outc = epi == kSwiglu ? TN / 2 : TN;
    p.tiles_m = (M + TM - 1) / TM;
    p.tiles_n = (N + outc - 1) / outc;
    const long long t = static_cast<long long>(p.tiles_m) * p.tiles_n;
    const int nk = (K + kTK - 1) / kTK;
    int s = 1;
    if (p.fm == 4 && t < 256 && nk >= 8) s = static_cast<int>(std::min<long long>((256 + t - 1) / t, nk / 4));
    s = std::max(1, s);
    const int kt_per = (nk + s - 1) / s;
    p.ksplit = std::max(1, kt_per) * kTK;
    p.splits = nk > 0 ? (nk + kt_per - 1) / kt_per : 1;
    // the partial layout of a split SwiGLU is the plain [M, 2N] product
    if (p.splits > 1 && epi == kSwiglu) p.tiles_n = (Nw + TN - 1) / TN;
    p.part_bytes = p.splits > 1 ? static_cast<size_t>(p.splits) * M * Nw * sizeof(float) : 0;
    return p;
}

// Whether the reduce of this launch can also write the RMSNorm of the new rows (a.nw set).
inline bool norm_fusable(const GemmArgs &a, int epi, const Plan &p)
{
    const auto a16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
    return a.nw != nullptr && a.nout != nullptr && epi == kAdd && p.splits > 1 && a.N % 8 == 0 && a.N <= 8192 &&
           a.ldo == a.N && a.ldr == a.N && a16(a.out) && a16(a.R) && a16(a.nw) && a16(a.nout);
}

// Whether the reduce of this launch can also write the conv requested through a.cu.
inline bool conv_fusable(const GemmArgs &a, int epi, const Plan &p)
{
    const auto a_n = [](const void *q, unsigned n) { return (reinterpret_cast<uintptr_t>(q) & (n - 1u)) == 0; };
    return a.cu != nullptr && a.cw != nullptr && a.c0 != nullptr && epi == kStore && (p.splits > 1 || p.stream) &&
           vec_ok(a, epi) &&
           a.cD > 0 && a.cD % 4 == 0 && a.cD <= a.N && a_n(a.cw, 16) && a_n(a.c0, 8) && a_n(a.cu, 8);
}

// Returns false (launching nothing) for a plan no kernel is built for.  *normed / *conved (if
// given) tell whether the RMSNorm requested through a.nw / the conv requested through a.cu
// were written (see norm_fusable, conv_fusable).
inline bool launch_gemm(GemmArgs a, int epi, const Plan &p, hipStream_t s, bool *normed = nullptr,
                        bool *conved = nullptr)
{
    if (normed != nullptr) *normed = false;
    if (conved != nullptr) *conved = false;
    if (!conv_fusable(a, epi, p)) a.cu = nullptr;
    if (p.fm == 8 && p.splits > 1 && !p.stream) return false;
    a.splits = p.splits;
    a.ksplit = p.ksplit;
    a.tiles_m = p.tiles_m;
    a.tiles_n = p.tiles_n;
    a.Nw = epi == kSwiglu ? 2 * a.N : a.N;
    a.group_m = 4;
    const int grid = p.tiles_m * p.tiles_n * p.splits;
    if (grid == 0) return true;
    const int kern_epi = p.splits > 1 ? kPartial : epi;
#define SAMBA_GEMM_LAUNCH(FM, FN, E) hipLaunchKernelGGL((gemm_kernel<2, 2, FM, FN, E>), dim3(grid), dim3(256), 0, s, a)
#define SAMBA_GEMM_LAUNCH8(E) hipLaunchKernelGGL((gemm_ring_kernel<4, 2, 4, 8, E, 2>), dim3(grid), dim3(512), 0, s, a)
    if (p.ring > 0) {
#define SAMBA_GEMM_RING128(S)                                                                                \
    switch (kern_epi) {                                                                                      \
    case kStore: hipLaunchKernelGGL((gemm_ring_kernel<2, 2, 4, 4, kStore, S>), dim3(grid), dim3(256), 0, s, a); break; \
    case kAdd: hipLaunchKernelGGL((gemm_ring_kernel<2, 2, 4, 4, kAdd, S>), dim3(grid), dim3(256), 0, s, a); break;     \
    case kSwiglu: hipLaunchKernelGGL((gemm_ring_kernel<2, 2, 4, 4, kSwiglu, S>), dim3(grid), dim3(256), 0, s, a); break; \
    default: hipLaunchKernelGGL((gemm_ring_kernel<2, 2, 4, 4, kPartial, S>), dim3(grid), dim3(256), 0, s, a); break; \
    }
        if (p.ring == 2) {
            SAMBA_GEMM_RING128(2)
        } else if (p.ring == 3) {
            SAMBA_GEMM_RING128(3)
        } else {
            SAMBA_GEMM_RING128(4)
        }
#undef SAMBA_GEMM_RING128
    } else if (p.stream) {
        bool ok = false;
#define SAMBA_GEMM_STREAM_SHAPE(FM, FN, NS)                                                          \
    if (p.fm == FM && p.fn == FN && p.ns == NS) {                                                    \
        ok = true;                                                                                   \
        switch (kern_epi) {                                                                          \
        case kStore: hipLaunchKernelGGL((gemm_stream_kernel<FM, FN, NS, kStore>), dim3(grid), dim3(256), 0, s, a); break; \
        case kAdd: hipLaunchKernelGGL((gemm_stream_kernel<FM, FN, NS, kAdd>), dim3(grid), dim3(256), 0, s, a); break;     \
        case kSwiglu: hipLaunchKernelGGL((gemm_stream_kernel<FM, FN, NS, kSwiglu>), dim3(grid), dim3(256), 0, s, a); break; \
        default: hipLaunchKernelGGL((gemm_stream_kernel<FM, FN, NS, kPartial>), dim3(grid), dim3(256), 0, s, a); break; \
        }                                                                                            \
    }
        SAMBA_GEMM_STREAM_SHAPE(4, 4, 2)
        SAMBA_GEMM_STREAM_SHAPE(4, 2, 2)
        SAMBA_GEMM_STREAM_SHAPE(2, 4, 2)
        SAMBA_GEMM_STREAM_SHAPE(2, 2, 2)
#undef SAMBA_GEMM_STREAM_SHAPE
        if (!ok) return false;
        if (conved != nullptr && p.splits == 1) *conved = a.cu != nullptr;
    } else if (p.fm == 8 && p.w8) {
        switch (kern_epi) {
        case kStore: SAMBA_GEMM_LAUNCH8(kStore); break;
        case kAdd: SAMBA_GEMM_LAUNCH8(kAdd); break;
        case kSwiglu: SAMBA_GEMM_LAUNCH8(kSwiglu); break;
        default: return false;
        }
    } else if (p.fm == 8) {
        return false;
    } else {
        switch (kern_epi) {
        case kStore: SAMBA_GEMM_LAUNCH(4, 4, kStore); break;
        case kAdd: SAMBA_GEMM_LAUNCH(4, 4, kAdd); break;
        case kSwiglu: SAMBA_GEMM_LAUNCH(4, 4, kSwiglu); break;
        default: SAMBA_GEMM_LAUNCH(4, 4, kPartial); break;
        }
    }
#undef SAMBA_GEMM_LAUNCH
#undef SAMBA_GEMM_LAUNCH8
    if (p.splits > 1 && norm_fusable(a, epi, p)) {
        switch ((a.N + 2047) / 2048) {
        case 1: hipLaunchKernelGGL(gemm_reduce_add_norm_kernel<1>, dim3(a.M), dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL(gemm_reduce_add_norm_kernel<2>, dim3(a.M), dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL(gemm_reduce_add_norm_kernel<3>, dim3(a.M), dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL(gemm_reduce_add_norm_kernel<4>, dim3(a.M), dim3(256), 0, s, a); break;
        }
        if (normed != nullptr) *normed = true;
    } else if (p.splits > 1) {
        const bool v4 = vec_ok(a, epi);
        if (conved != nullptr) *conved = a.cu != nullptr;
        const size_t n = static_cast<size_t>(a.M) * (v4 ? a.N / 4 : a.N);
        const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
#define SAMBA_GEMM_REDUCE(E)                                                                        \
    do {                                                                                            \
        if (v4)                                                                                     \
            hipLaunchKernelGGL((gemm_reduce_kernel<E, 4>), dim3(blocks), dim3(256), 0, s, a);       \
        else                                                                                        \
            hipLaunchKernelGGL((gemm_reduce_kernel<E, 1>), dim3(blocks), dim3(256), 0, s, a);       \
    } while (0)
        switch (epi) {
        case kStore: SAMBA_GEMM_REDUCE(kStore); break;
        case kAdd: SAMBA_GEMM_REDUCE(kAdd); break;
        default: SAMBA_GEMM_REDUCE(kSwiglu); break;
        }
#undef SAMBA_GEMM_REDUCE
    }
    return true;
}

}  // namespace gemm
}  // namespace samba
