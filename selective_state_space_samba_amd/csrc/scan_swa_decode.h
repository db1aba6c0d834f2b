// scan_swa_decode.h -- one decode step of sliding window attention over a ring-buffer KV
// cache (page 1, "The Sliding Window Attention (SWA) Layer": at position t a query reads the
// keys t-w .. t, so a sequence needs only the last w + 1 keys and values, whatever its length;
// with RoPE the cached keys are stored rotated at their own positions).
//
// The cache of a sequence and KV head is a ring of cap = w + 1 entries: position p lives in
// slot p mod cap, so after the new token's key and value are written the ring holds exactly
// the window.  A step is three launches:
//  1. store: rotate the new key at its position and write key and value into their slot;
//  2. attention, split over the keys (flash-decoding): a wave takes one (sequence, KV head,
//     key split) and the up-to-16 query heads of the group as the 16 columns of
//     S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16); keys are read straight
//     from the ring in the A-operand layout, values are transposed through the wave's own
//     LDS tile for O^T = V^T P^T; each split writes its unnormalised output, offset and sum;
//  3. combine: per (sequence, head), the splits' partial results are merged and stored.
#pragma once

#include "scan_swa.h"

namespace samba {

namespace swadec {
constexpr int kSplit = 4;   // key splits per (sequence, KV head); 8 and 16 measured slower
constexpr int kKeys = 64;   // keys per tile
constexpr int kMaxGroup = 16;
}  // namespace swadec

struct SwaDecArgs {
    int S, Hq, Hkv, dh, window, cap;
    float scale_log2;
    const void *q, *k, *v;  // new token: q [S][Hq][dh], k, v [S][Hkv][dh]
    int ldq, ldkv;          // row pitch of q and of k, v per sequence (0: contiguous)
    const int32_t *pos;     // [S] position of the new token (tokens before it in the sequence)
    uint16_t *kc, *vc;      // rings [S][Hkv][cap][dh], bfloat16, keys rotated
    void *out;              // [S][Hq][dh]
    float *part;            // workspace [S][Hq][kSplit][dh + 2]: O (unnormalised), offset, sum
    // fill (prefill -> ring)
    const int32_t *cu;
    int seqlen, total;
    float th_hi[swa::kMaxPairs], th_lo[swa::kMaxPairs];
};

namespace swadec {

__device__ inline void rotate8(const SwaDecArgs &a, int d, int pos, float *f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float p = static_cast<float>(pos);
        const float hi = a.th_hi[d / 2 + i];
        const float m = p * hi;
        const float err = __builtin_fmaf(p, hi, -m);
        const float fr = (m - __builtin_rintf(m)) + __builtin_fmaf(p, a.th_lo[d / 2 + i], err);
        const float c = __builtin_amdgcn_cosf(fr), s = __builtin_amdgcn_sinf(fr);
        const float x = f[2 * i], y = f[2 * i + 1];
        f[2 * i] = x * c - y * s;
        f[2 * i + 1] = __builtin_fmaf(x, s, y * c);
    }
}

__device__ inline void load8bf(const uint16_t *p, float *f)
{
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16lo(ws[i]);
        f[2 * i + 1] = bf16hi(ws[i]);
    }
}

__device__ inline uint4 pack8(const float *f)
{
    return make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
}

}  // namespace swadec

// 1. store the new token's rotated key and its value: grid S, 256 threads over (KV head, 8-element vector)
__global__ __launch_bounds__(256) void swa_dec_store_kernel(SwaDecArgs a)
{
    using namespace swadec;
    const int s = blockIdx.x;
    const int p = a.pos[s];
    if (p < 0) return;  // no token for this slot (caller data): nothing is written
    const int slot = p % a.cap;
    const int nvec = a.Hkv * a.dh / 8;
    for (int i = threadIdx.x; i < nvec; i += 256) {
        const int hk = i / (a.dh / 8), d = (i % (a.dh / 8)) * 8;
        const size_t ldkv = a.ldkv > 0 ? static_cast<size_t>(a.ldkv) : static_cast<size_t>(a.Hkv) * a.dh;
        const size_t src = static_cast<size_t>(s) * ldkv + static_cast<size_t>(hk) * a.dh + d;
        const size_t dst = ((static_cast<size_t>(s) * a.Hkv + hk) * a.cap + slot) * a.dh + d;
        float f[8];
        load8bf(static_cast<const uint16_t *>(a.k) + src, f);
        rotate8(a, d, p, f);
        *reinterpret_cast<uint4 *>(a.kc + dst) = pack8(f);
        *reinterpret_cast<uint4 *>(a.vc + dst) = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + src);
    }
}

// 2. attention over one key split: grid (kSplit, Hkv, S), 64 threads (one wave)
template <int kDh>
__global__ __launch_bounds__(64) void swa_dec_attn_kernel(SwaDecArgs a)
{
    using namespace swadec;
    using swa::bf16x8;
    using swa::f32x4;
    constexpr int kKS = kDh / 32, kDS = kDh / 16;
    constexpr int kVPitch = kKeys + 8;
    __shared__ __align__(16) uint16_t vs[kDh * kVPitch];
    const int sp = blockIdx.x, hk = blockIdx.y, s = blockIdx.z;
    const int l = threadIdx.x, g = l >> 4, c16 = l & 15;
    const int G = a.Hq / a.Hkv;
    const int pos = a.pos[s];
    const int lo = max(0, pos - a.window);
    const int nkeys = pos >= 0 ? pos - lo + 1 : 0;
    const int ntile = (nkeys + kKeys - 1) / kKeys;
    const int tps = (ntile + kSplit - 1) / kSplit;
    const int tb = sp * tps, te = min(ntile, tb + tps);
    const size_t ring = (static_cast<size_t>(s) * a.Hkv + hk) * a.cap;  // first entry of this ring

    // query vector c16 = head hk * G + c16 (zeros past the group), rotated and scaled,
    // split into high and low bfloat16 parts
    bf16x8 qf[kKS], ql[kKS];
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
        float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        const int d = 32 * kk + 8 * g;
        if (c16 < G && pos >= 0) {
            const size_t ldq = a.ldq > 0 ? static_cast<size_t>(a.ldq) : static_cast<size_t>(a.Hq) * kDh;
            load8bf(static_cast<const uint16_t *>(a.q) + static_cast<size_t>(s) * ldq +
                        static_cast<size_t>(hk * G + c16) * kDh + d, f);
            rotate8(a, d, pos, f);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f[e] *= a.scale_log2;
            qf[kk][e] = static_cast<__bf16>(f[e]);
            ql[kk][e] = static_cast<__bf16>(f[e] - static_cast<float>(qf[kk][e]));
        }
    }
    f32x4 o[kDS];
#pragma unroll
    for (int i = 0; i < kDS; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -1e30f, l_run = 0.0f;

    for (int ti = tb; ti < te; ++ti) {
        const int p0 = lo + ti * kKeys;  // position of the tile's first key
        // stage V^T (this wave only): a lane transposes blocks of 4 keys x 8 elements
        {
            constexpr int kBlocks = (kKeys / 4) * (kDh / 8);
#pragma unroll
            for (int bi = 0; bi < kBlocks / 64; ++bi) {
                // element groups are the fast index so that a lane group reads 128 contiguous
                // bytes of a ring entry; the transposed map (key groups fast) removes the V^T
                // write bank conflicts but halves the read segments and measured 9 % slower:
                // this kernel is bound by reading the rings
                const int blk = bi * 64 + l;
                const int kg = blk / (kDh / 8), d = (blk % (kDh / 8)) * 8;
                uint32_t w[4][4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = min(p0 + 4 * kg + r, pos);  // keys past pos: clamped, masked below
                    const uint4 v4 = *reinterpret_cast<const uint4 *>(a.vc + (ring + p % a.cap) * kDh + d);
                    w[r][0] = v4.x;
                    w[r][1] = v4.y;
                    w[r][2] = v4.z;
                    w[r][3] = v4.w;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    *reinterpret_cast<uint2 *>(&vs[(d + 2 * e) * kVPitch + 4 * kg]) =
                        make_uint2(__builtin_amdgcn_perm(w[1][e], w[0][e], 0x05040100u),
                                   __builtin_amdgcn_perm(w[3][e], w[2][e], 0x05040100u));
                    *reinterpret_cast<uint2 *>(&vs[(d + 2 * e + 1) * kVPitch + 4 * kg]) =
                        make_uint2(__builtin_amdgcn_perm(w[1][e], w[0][e], 0x07060302u),
                                   __builtin_amdgcn_perm(w[3][e], w[2][e], 0x07060302u));
                }
            }
        }
        // S^T: keys straight from the ring in the A-operand layout
        f32x4 sc[kKeys / 16];
#pragma unroll
        for (int st = 0; st < kKeys / 16; ++st) {
            const int p = min(p0 + 16 * st + c16, pos);
            const uint16_t *krow = a.kc + (ring + p % a.cap) * kDh;
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < kKS; ++kk) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(krow + 32 * kk + 8 * g);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[kk], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[kk], acc, 0, 0, 0);
            }
            sc[st] = acc;
        }
        if (p0 + kKeys - 1 > pos) {  // the tile holding pos: keys past it do not exist
#pragma unroll
            for (int st = 0; st < kKeys / 16; ++st)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sc[st][e] = (p0 + 16 * st + 4 * g + e > pos) ? -__builtin_inff() : sc[st][e];
        }
        float mt = -1e30f;
#pragma unroll
        for (int st = 0; st < kKeys / 16; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) mt = __builtin_fmaxf(mt, sc[st][e]);
        mt = __builtin_fmaxf(mt, __shfl_xor(mt, 16));
        mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
        if (__any(mt > m_run + 8.0f)) {
            const float m_new = __builtin_fmaxf(m_run, mt);
            const float alpha = hw_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < kDS; ++i) o[i] *= alpha;
        }
        // probabilities in two bfloat16 parts (the value products are cheap here: the step
        // is bound by reading the rings)
        bf16x8 pb[kKeys / 32], pl[kKeys / 32];
#pragma unroll
        for (int st = 0; st < kKeys / 16; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pr = hw_exp2(sc[st][e] - m_run);
                l_run += pr;
                const __bf16 hi = static_cast<__bf16>(pr);
                pb[st / 2][(st & 1) * 4 + e] = hi;
                pl[st / 2][(st & 1) * 4 + e] = static_cast<__bf16>(pr - static_cast<float>(hi));
            }
        __syncthreads();  // one-wave workgroup: the V^T tile is complete
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) {
            const uint16_t *vrow = &vs[(16 * ds + c16) * kVPitch];
#pragma unroll
            for (int kk = 0; kk < kKeys / 32; ++kk) {
                const uint2 lo2 = *reinterpret_cast<const uint2 *>(vrow + 32 * kk + 4 * g);
                const uint2 hi2 = *reinterpret_cast<const uint2 *>(vrow + 32 * kk + 16 + 4 * g);
                const uint4 w = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
                o[ds] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), pb[kk], o[ds], 0, 0, 0);
                o[ds] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), pl[kk], o[ds], 0, 0, 0);
            }
        }
        __syncthreads();  // the tile is read before the next one is staged
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (c16 < G) {
        float *pp = a.part + ((static_cast<size_t>(s) * a.Hq + hk * G + c16) * kSplit + sp) * (kDh + 2);
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds)
            *reinterpret_cast<float4 *>(pp + 16 * ds + 4 * g) = make_float4(o[ds][0], o[ds][1], o[ds][2], o[ds][3]);
        if (g == 0) {
            pp[kDh] = m_run;
            pp[kDh + 1] = l_run;
        }
    }
}

// 3. combine the splits: grid S * Hq, dh threads
__global__ __launch_bounds__(256) void swa_dec_combine_kernel(SwaDecArgs a)
{
    using namespace swadec;
    const int sh = blockIdx.x;
    const int d = threadIdx.x;
    if (d >= a.dh) return;
    const float *pp = a.part + static_cast<size_t>(sh) * kSplit * (a.dh + 2);
    float M = -1e30f;
    for (int k = 0; k < kSplit; ++k) M = __builtin_fmaxf(M, pp[k * (a.dh + 2) + a.dh]);
    float num = 0.0f, den = 0.0f;
    for (int k = 0; k < kSplit; ++k) {
        const float w = hw_exp2(pp[k * (a.dh + 2) + a.dh] - M);
        num = __builtin_fmaf(w, pp[k * (a.dh + 2) + d], num);
        den = __builtin_fmaf(w, pp[k * (a.dh + 2) + a.dh + 1], den);
    }
    IoBf16::st(a.out, static_cast<size_t>(sh) * a.dh + d, den > 0.0f ? num / den : 0.0f);
}

// Prefill -> rings: grid (S, ceil(cap / 4)), 256 threads; each sequence's last min(L, cap)
// tokens are written rotated (keys) and as they are (values) into slot position mod cap.
__global__ __launch_bounds__(256) void swa_kv_fill_kernel(SwaDecArgs a)
{
    using namespace swadec;
    const int s = blockIdx.x;
    int t0, t1;
    if (a.cu != nullptr) {
        t0 = min(max(a.cu[s], 0), a.total);
        t1 = min(max(a.cu[s + 1], t0), a.total);
    } else {
        t0 = s * a.seqlen;
        t1 = t0 + a.seqlen;
    }
    const int L = t1 - t0;
    const int first = max(0, L - a.cap);  // oldest position kept
    const int nvec = a.Hkv * a.dh / 8;
    const int per = 4;  // positions per workgroup
    for (int i = threadIdx.x; i < per * nvec; i += 256) {
        const int p = first + blockIdx.y * per + i / nvec;
        if (p >= L) continue;
        const int vi = i % nvec;
        const int hk = vi / (a.dh / 8), d = (vi % (a.dh / 8)) * 8;
        const size_t src = (static_cast<size_t>(t0 + p) * a.Hkv + hk) * a.dh + d;
        const size_t dst = ((static_cast<size_t>(s) * a.Hkv + hk) * a.cap + p % a.cap) * a.dh + d;
        float f[8];
        load8bf(static_cast<const uint16_t *>(a.k) + src, f);
        rotate8(a, d, p, f);
        *reinterpret_cast<uint4 *>(a.kc + dst) = pack8(f);
        *reinterpret_cast<uint4 *>(a.vc + dst) = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + src);
    }
}

inline size_t swa_decode_workspace_bytes(int S, int Hq, int dh)
{
    return (static_cast<size_t>(S) * Hq * swadec::kSplit * (dh + 2) * sizeof(float) + 255) / 256 * 256;
}

inline void swa_dec_set_theta(SwaDecArgs &a, double base)
{
    for (int i = 0; i < a.dh / 2; ++i) {
        const double th = std::pow(base, -2.0 * i / a.dh) / (2.0 * 3.14159265358979323846);
        const float hi = static_cast<float>(th);
        a.th_hi[i] = hi;
        a.th_lo[i] = static_cast<float>(th - static_cast<double>(hi));
    }
}

inline void launch_swa_decode(const SwaDecArgs &a, hipStream_t stream)
{
    using namespace swadec;
    swa_dec_store_kernel<<<a.S, 256, 0, stream>>>(a);
    const dim3 g(kSplit, a.Hkv, a.S);
    if (a.dh == 64)
        swa_dec_attn_kernel<64><<<g, 64, 0, stream>>>(a);
    else
        swa_dec_attn_kernel<128><<<g, 64, 0, stream>>>(a);
    swa_dec_combine_kernel<<<a.S * a.Hq, 256, 0, stream>>>(a);
}

inline void launch_swa_kv_fill(const SwaDecArgs &a, hipStream_t stream)
{
    const dim3 g(a.S, (a.cap + 3) / 4);
    swa_kv_fill_kernel<<<g, 256, 0, stream>>>(a);
}

}  // namespace samba
