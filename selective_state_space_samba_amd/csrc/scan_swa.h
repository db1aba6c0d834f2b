// scan_swa.h -- sliding window attention of the Samba layer stack (page 1, "The Sliding
// Window Attention (SWA) Layer": causal attention over the keys at positions t-w .. t of
// the same sequence, RoPE with base 10000 on queries and keys, grouped KV heads).
//
// The one dense contraction of the model family that the scan library serves, so it runs
// on the matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//  * a workgroup owns 64 query rows of one query head (16 rows per wave) and walks the
//    key tiles of 64 that the rows' windows cover (w / 64 + 1 tiles);
//  * a wave computes S^T = K Q^T per 16-key sub-tile, so each lane holds 4 consecutive keys
//    of one query row: the row's softmax statistics need only two cross-lane steps, the
//    rescale of the output is one factor per lane, and the probabilities are already in
//    the B-operand layout of O^T = V^T P^T (the contraction runs over the keys in the
//    order the S^T layout leaves them, and V^T is read from LDS in that same order);
//  * K (rotated once by a pre-pass, bfloat16) and V^T tiles are staged through LDS, double
//    buffered, the next tile's loads in flight while the current one is computed;
//  * the queries are rotated on load; all RoPE angles are reduced exactly to revolutions
//    (position times a double-float theta / 2 pi) before the hardware sin / cos, so
//    positions of any size keep full accuracy.
#pragma once

#include "scan_common.h"

namespace samba {

namespace swa {

constexpr int kRows = 64;   // query rows per workgroup and row block of its waves (16 per wave)
// Row blocks per wave: a wave takes kRB blocks of 16 query rows, so every K and V^T fragment
// it reads from LDS feeds kRB sets of MFMAs and a staged key tile serves 64 kRB rows.
// head_dim 64: two; head_dim 128: one (no registers left for a second).
template <int kDh>
constexpr int row_blocks() { return kDh == 64 ? 2 : 1; }
inline int rows_per_workgroup(int dh) { return kRows * (dh == 64 ? row_blocks<64>() : row_blocks<128>()); }
constexpr int kKeys = 64;   // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxPairs = 128;  // head_dim <= 256

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

}  // namespace swa

struct SwaArgs {
    int nseq, seqlen;   // seqlen: per sequence (fixed) or the longest (packed)
    const int32_t *cu;  // packed offsets or nullptr
    int total;
    int Hq, Hkv, dh, window;
    int nrb;            // row blocks per sequence slot = ceil(seqlen / rows_per_workgroup(dh))
    float scale_log2;   // log2(e) / sqrt(dh)
    const void *q, *k, *v;
    void *out;
    uint16_t *krot;     // workspace: rotated keys [total][Hkv][dh] bfloat16
    float th_hi[swa::kMaxPairs], th_lo[swa::kMaxPairs];  // theta_i / 2 pi as hi + lo
};

namespace swa {

__device__ inline void seq_bounds(const SwaArgs &a, int s, int &t0, int &t1)
{
    if (a.cu != nullptr) {
        t0 = min(max(a.cu[s], 0), a.total);
        t1 = min(max(a.cu[s + 1], t0), a.total);
    } else {
        t0 = s * a.seqlen;
        t1 = t0 + a.seqlen;
    }
}

// cos / sin of pos * theta_i: the product is formed exactly as hi + err + lo terms and
// reduced to a fraction of a revolution before v_cos_f32 / v_sin_f32 (which take
// revolutions).
__device__ inline void rope_cs(const SwaArgs &a, int i, int pos, float &c, float &s)
{
    const float p = static_cast<float>(pos);
    const float hi = a.th_hi[i];
    const float m = p * hi;
    const float err = __builtin_fmaf(p, hi, -m);
    const float fr = (m - __builtin_rintf(m)) + __builtin_fmaf(p, a.th_lo[i], err);
    c = __builtin_amdgcn_cosf(fr);
    s = __builtin_amdgcn_sinf(fr);
}

// 8 consecutive elements (d .. d+7) of a head vector as floats.
template <class Io>
__device__ inline void load8(const void *base, size_t off, float *f)
{
    if constexpr (sizeof(typename Io::T) == 2) {
        const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16lo(ws[i]);
            f[2 * i + 1] = bf16hi(ws[i]);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off);
        const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off + 4);
        f[0] = a.x;
        f[1] = a.y;
        f[2] = a.z;
        f[3] = a.w;
        f[4] = b.x;
        f[5] = b.y;
        f[6] = b.z;
        f[7] = b.w;
    }
}

// Rotates the 4 pairs of 8 consecutive elements starting at element d (even) at position pos.
__device__ inline void rotate8(const SwaArgs &a, int d, int pos, float *f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float c, s;
        rope_cs(a, d / 2 + i, pos, c, s);
        const float x = f[2 * i], y = f[2 * i + 1];
        f[2 * i] = x * c - y * s;
        f[2 * i + 1] = __builtin_fmaf(x, s, y * c);
    }
}

}  // namespace swa

// ---------------------------------------------------------------- key rotation pre-pass
// grid (nseq * nruns), 256 threads: each thread rotates 8-element vectors of the keys of a
// run of 64 tokens of one sequence (positions count from the sequence start).
template <class Io>
__global__ __launch_bounds__(256) void swa_rotate_keys_kernel(SwaArgs a, int nruns)
{
    using namespace swa;
    const int s = blockIdx.x / nruns, r = blockIdx.x - s * nruns;
    int t0, t1;
    seq_bounds(a, s, t0, t1);
    const int nvec = a.Hkv * a.dh / 8;  // vectors per token
    const int tb = t0 + r * 64, te = min(tb + 64, t1);
    for (int i = threadIdx.x; i < (te - tb) * nvec; i += 256) {
        const int t = tb + i / nvec, vi = i - (i / nvec) * nvec;
        const int d = (vi * 8) % a.dh;
        float f[8];
        const size_t off = static_cast<size_t>(t) * a.Hkv * a.dh + static_cast<size_t>(vi) * 8;
        load8<Io>(a.k, off, f);
        rotate8(a, d, t - t0, f);
        *reinterpret_cast<uint4 *>(a.krot + off) =
            make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
    }
}

// ---------------------------------------------------------------- attention
// grid nseq * Hq * ceil(seqlen / 64) (one dimension, see the mapping below), 256 threads.
template <class Io, int kDh>
// head_dim 64: the register budget of three waves per SIMD (168 registers, no spill; three
// workgroups of 34 KB LDS per CU) -- 18 % faster than the two the unconstrained allocation
// (221 registers) leaves; head_dim 128 does not fit three.
__global__ __launch_bounds__(swa::kThreads, kDh == 64 ? 3 : 2) void swa_attention_kernel(SwaArgs a)
{
    using namespace swa;
    using T = typename Io::T;
    constexpr int kKS = kDh / 32;         // k-steps of S^T = K Q^T
    constexpr int kDS = kDh / 16;         // d sub-tiles of O^T
    // K rows are unpadded (kDh elements); 16-byte chunk q of key row r sits at chunk
    // q ^ kswz(r), so that the 16 rows a fragment read touches (and the two rows a 16-lane
    // group of the staging writes fills) fall on distinct banks
    constexpr int kKPitch = kDh;
    auto kswz = [](int r) { return kDh == 64 ? ((r >> 1) & 7) : (r & 15); };
    constexpr int kVPitch = kKeys + 8;    // LDS pitch of a V^T row (bf16)
    __shared__ __align__(16) uint16_t ks[2][kKeys * kKPitch];
    __shared__ __align__(16) uint16_t vs[2][kDh * kVPitch];

    // Workgroup -> (sequence, query head, row block).  The hardware deals workgroups to the
    // 8 XCDs round-robin; each XCD gets one contiguous range of the logical order
    // (sequence, KV head, row block, query head of the group), so an XCD's L2 sees the 8
    // query heads that share a key tile next to each other and neighbouring row blocks
    // whose windows overlap.
    int rb, h, s;
    {
        const int W = gridDim.x, i = blockIdx.x;
        const int x = i & 7, j = i >> 3;
        const int logical = x * (W >> 3) + min(x, W & 7) + j;
        const int G = a.Hq / a.Hkv, nrb = a.nrb;
        const int hg = logical % G;
        const int rest = logical / G;
        rb = rest % nrb;
        const int rest2 = rest / nrb;
        h = (rest2 % a.Hkv) * G + hg;
        s = rest2 / a.Hkv;
    }
    int t0, t1;
    seq_bounds(a, s, t0, t1);
    const int L = t1 - t0;
    constexpr int kRB = row_blocks<kDh>();
    const int R0 = rb * kRows * kRB;
    if (R0 >= L) return;  // uniform over the workgroup
    const int hk = h / (a.Hq / a.Hkv);
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
    const int g = l >> 4, c16 = l & 15;
    // this lane's query rows (positions in the sequence): row c16 of the wave's blocks
    const int rw0 = R0 + wave * 16 * kRB;
    int row[kRB];
#pragma unroll
    for (int b = 0; b < kRB; ++b) row[b] = rw0 + 16 * b + c16;

    // queries of the wave's 16 rows as the B operand of S^T = K Q^T: lane (g, c16) holds
    // row c16, elements 32 ks + 8 g .. +7, rotated
    // (high and low bfloat16 parts: the scores are formed as K Qhi + K Qlo, so rounding the
    // rotated queries to bfloat16 does not move them; the keys are rounded once, as
    // FlashAttention-2's bfloat16 operands are)
    bf16x8 qf[kRB][kKS], ql[kRB][kKS];
#pragma unroll
    for (int b = 0; b < kRB; ++b) {
        const int rowc = min(row[b], L - 1);
#pragma unroll
        for (int kk = 0; kk < kKS; ++kk) {
            const int d = 32 * kk + 8 * g;
            float f[8];
            load8<Io>(a.q, (static_cast<size_t>(t0 + rowc) * a.Hq + h) * kDh + d, f);
            rotate8(a, d, rowc, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                f[e] *= a.scale_log2;  // scores come out in log2 units
                qf[b][kk][e] = static_cast<__bf16>(f[e]);
                ql[b][kk][e] = static_cast<__bf16>(f[e] - static_cast<float>(qf[b][kk][e]));
            }
        }
    }

    // key tiles covering [R0 - window, R0 + 64 kRB - 1] within the sequence
    const int klo = max(0, R0 - a.window);
    const int kt0 = klo / kKeys * kKeys;
    const int khi = min(L, R0 + kRows * kRB);  // exclusive
    const int ntiles = (khi - kt0 + kKeys - 1) / kKeys;

    // staging: threads 0..127 move the V tile, transposing it to V^T in registers (a thread
    // reads 4 keys x 8 elements and writes 8 rows of 4 keys); threads 128..255 move the K
    // tile (rotated keys) as 16-byte pieces.  Consecutive V-staging lanes take consecutive
    // 4-key groups (key group = lane % 16): their 8-byte V^T writes then fall on distinct
    // banks of the 144-byte-pitch rows (with the element group as the fast index, four lanes
    // of a half-wave shared a bank pair: 60 % of the kernel's LDS cycles were conflicts).
    constexpr int kKPieces = kKeys * kDh / 8;          // 16-byte pieces of the K tile
    constexpr int kKPer = kKPieces / 128;              // per K-staging thread
    constexpr int kVBlocks = (kKeys / 4) * (kDh / 8);  // 4-key x 8-element blocks of V
    constexpr int kVPer = kVBlocks / 128;              // per V-staging thread
    static_assert(kKPieces % 128 == 0 && kVBlocks % 128 == 0, "staging split");
    const bool vstager = tid < 128;
    const int st_id = tid & 127;
    uint4 sreg[kVPer * 4 > kKPer ? kVPer * 4 : kKPer];
    auto fetch = [&](int kt) {
        if (vstager) {
#pragma unroll
            for (int i = 0; i < kVPer; ++i) {
                const int bi = i * 128 + st_id;
                const int kg = bi % (kKeys / 4), d = (bi / (kKeys / 4)) * 8;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kk = min(kt + 4 * kg + r, L - 1);  // keys past the end: clamped, masked later
                    sreg[i * 4 + r] = *reinterpret_cast<const uint4 *>(
                        static_cast<const uint16_t *>(a.v) + (static_cast<size_t>(t0 + kk) * a.Hkv + hk) * kDh + d);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kKPer; ++i) {
                const int pi = i * 128 + st_id;
                const int key = pi / (kDh / 8), d = (pi % (kDh / 8)) * 8;
                const int kk = min(kt + key, L - 1);
                sreg[i] = *reinterpret_cast<const uint4 *>(a.krot + (static_cast<size_t>(t0 + kk) * a.Hkv + hk) * kDh + d);
            }
        }
    };
    auto stage = [&](int buf) {
        if (vstager) {
#pragma unroll
            for (int i = 0; i < kVPer; ++i) {
                const int bi = i * 128 + st_id;
                const int kg = bi % (kKeys / 4), d = (bi / (kKeys / 4)) * 8;
                const uint32_t w0[4] = {sreg[i * 4].x, sreg[i * 4].y, sreg[i * 4].z, sreg[i * 4].w};
                const uint32_t w1[4] = {sreg[i * 4 + 1].x, sreg[i * 4 + 1].y, sreg[i * 4 + 1].z, sreg[i * 4 + 1].w};
                const uint32_t w2[4] = {sreg[i * 4 + 2].x, sreg[i * 4 + 2].y, sreg[i * 4 + 2].z, sreg[i * 4 + 2].w};
                const uint32_t w3[4] = {sreg[i * 4 + 3].x, sreg[i * 4 + 3].y, sreg[i * 4 + 3].z, sreg[i * 4 + 3].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {  // elements d + 2e (low halves) and d + 2e + 1 (high halves)
                    const uint2 lo = make_uint2(__builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u),
                                                __builtin_amdgcn_perm(w3[e], w2[e], 0x05040100u));
                    const uint2 hi = make_uint2(__builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u),
                                                __builtin_amdgcn_perm(w3[e], w2[e], 0x07060302u));
                    *reinterpret_cast<uint2 *>(&vs[buf][(d + 2 * e) * kVPitch + 4 * kg]) = lo;
                    *reinterpret_cast<uint2 *>(&vs[buf][(d + 2 * e + 1) * kVPitch + 4 * kg]) = hi;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kKPer; ++i) {
                const int pi = i * 128 + st_id;
                const int key = pi / (kDh / 8), d = (pi % (kDh / 8)) * 8;
                *reinterpret_cast<uint4 *>(&ks[buf][key * kKPitch + (((d >> 3) ^ kswz(key)) << 3)]) = sreg[i];
            }
        }
    };

    f32x4 o[kRB][kDS];
    float m_run[kRB], l_run[kRB];  // exponent offset (log2 units) and this lane's share of the sum
#pragma unroll
    for (int b = 0; b < kRB; ++b) {
#pragma unroll
        for (int i = 0; i < kDS; ++i) o[b][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        m_run[b] = -1e30f;
        l_run[b] = 0.0f;
    }

    fetch(kt0);
    stage(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        const int kt = kt0 + it * kKeys;
        if (it + 1 < ntiles) fetch(kt + kKeys);
        // S^T for the 4 sub-tiles of 16 keys: lane holds keys kt + 16 st + 4 g + e of row c16 of
        // each of its blocks; one K fragment read serves every block
        f32x4 sc[kRB][kKeys / 16];
#pragma unroll
        for (int st = 0; st < kKeys / 16; ++st) {
            f32x4 acc[kRB];
#pragma unroll
            for (int b = 0; b < kRB; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < kKS; ++kk) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
                    &ks[buf][(16 * st + c16) * kKPitch + (((4 * kk + g) ^ kswz(16 * st + c16)) << 3)]);
#pragma unroll
                for (int b = 0; b < kRB; ++b) {
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[b][kk], acc[b], 0, 0, 0);
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[b][kk], acc[b], 0, 0, 0);
                }
            }
#pragma unroll
            for (int b = 0; b < kRB; ++b) sc[b][st] = acc[b];
        }
        // mask: only tiles that cross a window edge, the diagonal or the sequence end for
        // some row of the wave (a wave-uniform test), then element selects
        if (kt < rw0 + 16 * kRB - 1 - a.window || kt + kKeys - 1 > rw0 || kt + kKeys > L) {
#pragma unroll
            for (int b = 0; b < kRB; ++b)
#pragma unroll
                for (int st = 0; st < kKeys / 16; ++st) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = kt + 16 * st + 4 * g + e;
                        sc[b][st][e] = (key > row[b] || key < row[b] - a.window || key >= L) ? -__builtin_inff() : sc[b][st][e];
                    }
                }
        }
        // probabilities, as the B operand of O^T = V^T P^T (k-step kk = sub-tiles 2kk, 2kk+1)
        bf16x8 pb[kRB][kKeys / 32];
#pragma unroll
        for (int b = 0; b < kRB; ++b) {
            float mt = -1e30f;
#pragma unroll
            for (int st = 0; st < kKeys / 16; ++st)
#pragma unroll
                for (int e = 0; e < 4; ++e) mt = __builtin_fmaxf(mt, sc[b][st][e]);
            mt = __builtin_fmaxf(mt, __shfl_xor(mt, 16));
            mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
            // The exponent offset m_run only moves when some row of the block would otherwise
            // see probabilities above 2^8 (the output and sum are then rescaled); between moves
            // the probabilities stay in (0, 256], which bfloat16 and the fp32 sums carry
            // exactly as well.
            if (__any(mt > m_run[b] + 8.0f)) {
                const float m_new = __builtin_fmaxf(m_run[b], mt);
                const float alpha = hw_exp2(m_run[b] - m_new);
                m_run[b] = m_new;
                l_run[b] *= alpha;
#pragma unroll
                for (int i = 0; i < kDS; ++i) o[b][i] *= alpha;
            }
            const float m_new = m_run[b];
#pragma unroll
            for (int st = 0; st < kKeys / 16; ++st) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = hw_exp2(sc[b][st][e] - m_new);
                    l_run[b] += p;
                    pb[b][st / 2][(st & 1) * 4 + e] = static_cast<__bf16>(p);
                }
            }
        }
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) {
            const uint16_t *vrow = &vs[buf][(16 * ds + c16) * kVPitch];
#pragma unroll
            for (int kk = 0; kk < kKeys / 32; ++kk) {
                // keys 32 kk + 4 g .. +3 and 32 kk + 16 + 4 g .. +3, in the order of pb
                const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + 32 * kk + 4 * g);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 32 * kk + 16 + 4 * g);
                const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
                for (int b = 0; b < kRB; ++b)
                    o[b][ds] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[b][kk], o[b][ds], 0, 0, 0);
            }
        }
        if (it + 1 < ntiles) {
            stage(buf ^ 1);  // the other buffer was last read in the previous iteration
        }
        __syncthreads();
    }
    // normalise and store: lane holds O[row c16][16 ds + 4 g + e] of each block
#pragma unroll
    for (int b = 0; b < kRB; ++b) {
        float lsum = l_run[b];
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        if (row[b] < L) {
            const float inv = 1.0f / lsum;
            T *op = static_cast<T *>(a.out) + (static_cast<size_t>(t0 + row[b]) * a.Hq + h) * kDh;
#pragma unroll
            for (int ds = 0; ds < kDS; ++ds) {
                const int d = 16 * ds + 4 * g;
                if constexpr (sizeof(T) == 2) {
                    *reinterpret_cast<uint2 *>(op + d) = make_uint2(pack_bf16(o[b][ds][0] * inv, o[b][ds][1] * inv),
                                                                    pack_bf16(o[b][ds][2] * inv, o[b][ds][3] * inv));
                } else {
                    *reinterpret_cast<float4 *>(op + d) = make_float4(o[b][ds][0] * inv, o[b][ds][1] * inv,
                                                                      o[b][ds][2] * inv, o[b][ds][3] * inv);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- host side
inline size_t swa_workspace_bytes(int total, int Hkv, int dh)
{
    return (static_cast<size_t>(total) * Hkv * dh * sizeof(uint16_t) + 255) / 256 * 256;
}

inline void swa_set_theta(SwaArgs &a, double base)
{
    for (int i = 0; i < a.dh / 2; ++i) {
        const double th = std::pow(base, -2.0 * i / a.dh) / (2.0 * 3.14159265358979323846);
        const float hi = static_cast<float>(th);
        a.th_hi[i] = hi;
        a.th_lo[i] = static_cast<float>(th - static_cast<double>(hi));
    }
}

// bfloat16 I/O only: the matrix-core operands are bfloat16, so float32 inputs would be
// rounded to bfloat16 anyway and could not meet a float32 tolerance.
inline void launch_swa(SwaArgs a, hipStream_t stream)
{
    using namespace swa;
    const int nruns = std::max(1, (a.seqlen + 63) / 64);
    const dim3 gr(static_cast<unsigned>(a.nseq) * nruns);
    swa_rotate_keys_kernel<IoBf16><<<gr, 256, 0, stream>>>(a, nruns);
    const int rows = rows_per_workgroup(a.dh);
    a.nrb = (a.seqlen + rows - 1) / rows;
    const size_t W = static_cast<size_t>(a.nrb) * a.Hq * a.nseq;
    if (W == 0) return;
    const dim3 ga(static_cast<unsigned>(W));
    if (a.dh == 64)
        swa_attention_kernel<IoBf16, 64><<<ga, kThreads, 0, stream>>>(a);
    else
        swa_attention_kernel<IoBf16, 128><<<ga, kThreads, 0, stream>>>(a);
}

}  // namespace samba
