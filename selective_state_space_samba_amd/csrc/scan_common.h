// scan_common.h -- shared device helpers for the selective-scan kernels (gfx950).
//
// Arithmetic is float32 on the hardware transcendental units: v_exp_f32 (2^x),
// v_log_f32 (log2 x) and v_rcp_f32 (1/x).  Natural-base quantities are carried in log2
// units where that saves a multiply: with Lg = softplus(a) * log2(e) one has
// exp(Delta * A) = 2^(Lg * A) and Delta = Lg * ln 2.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace samba {

constexpr int kMaxState = 16;  // d_state = 16 on every configuration of the pages
constexpr int kConvK = 4;      // short-conv kernel size k = 4

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Argument block shared by every scan kernel.  Pointers are device pointers.
struct ScanArgs {
    int nseq;            // sequences (batch)
    int seqlen;          // tokens per sequence (fixed-length) or max_seqlen (varlen)
    const int32_t *cu;   // varlen offsets [nseq + 1] or nullptr (fixed length)
    int total;           // tokens in the packed arrays (varlen); offsets are clamped to it
    int D;               // d_inner
    int N;               // d_state (<= kMaxState)
    const void *x, *dt, *B, *C, *z;
    int ldx, ldbc;       // decode only: row pitch of x and z, of B and C (0: contiguous)
    const float *A, *Dskip, *dt_bias, *conv_w, *conv_b;
    const float *h0;
    const void *conv0;
    void *out;
    float *h_final;
    void *conv_final;
    // Decode only: the conv history is a ring [seq][3][d_inner] whose slot (head + k) mod 3
    // holds x_{t-3+k}, head = head_in[seq] (any int; taken mod 3).  A step reads the three
    // slots and writes the new input into slot head (the oldest); head_out[seq] (nullable)
    // receives (head + 1) mod 3.  head_in == nullptr: the history is stored oldest first.
    const int32_t *head_in;
    int32_t *head_out;
    // Prefill / varlen: x holds u = SiLU(conv(x)), computed beforehand; the conv, its
    // parameters, conv0 and conv_final are not used.
    bool u_in;
};

// Ring slot of the history entry k (0 = oldest) for a head value from device memory.
__device__ inline int ring_slot(int head, int k)
{
    const int h = head % 3;
    return (h + (h < 0 ? 3 : 0) + k) % 3;
}

// Token range [t0, t1) of sequence s.  Varlen offsets are device data supplied by the
// caller; they are clamped into [0, total] so that malformed offsets can never address
// memory outside the packed arrays.
__device__ inline void seq_range(const ScanArgs &a, int s, size_t &t0, size_t &t1)
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

// ---------------------------------------------------------------- I/O element types
struct IoF32 {
    using T = float;
    __device__ static inline float ld(const void *p, size_t i) { return static_cast<const float *>(p)[i]; }
    __device__ static inline void st(void *p, size_t i, float v) { static_cast<float *>(p)[i] = v; }
};

struct IoBf16 {
    using T = uint16_t;
    __device__ static inline float ld(const void *p, size_t i)
    {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
    }
    // Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
    __device__ static inline void st(void *p, size_t i, float v)
    {
        static_cast<uint16_t *>(p)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    }
};

// s_waitcnt immediate that waits until at most n vector-memory operations of this wave are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their
// maxima, i.e. not waited for).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// A workgroup barrier with no memory fence: the compiler keeps every memory access on its
// side of it (the empty asm statements clobber memory) but adds no wait of its own, so loads
// into LDS issued before it stay in flight.  (__syncthreads() carries a workgroup fence that
// waits for all of them.)
__device__ inline void barrier_no_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Raw buffer access: a wave-uniform 128-bit resource (base, byte range) in SGPRs plus a
// 32-bit per-lane byte offset.  The hardware returns 0 for loads and drops stores whose
// offset falls outside the range, so a resource built from the exact extent of an
// array bounds every access to it.
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer descriptor flags

// base and bytes must be the same in every lane of the wave.  They are read from the
// first active lane: a value the compiler happens to compute in vector registers would
// otherwise make it wrap every access in a loop over the distinct values.
__device__ inline Rsrc make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    void *ub = reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0),
                                             static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), kRsrcWord3);
}
__device__ inline void buf_ld(Rsrc r, uint32_t boff, float &v)
{
    v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, boff, 0, 0));
}
__device__ inline void buf_ld(Rsrc r, uint32_t boff, uint16_t &v)
{
    v = __builtin_amdgcn_raw_buffer_load_b16(r, boff, 0, 0);
}
__device__ inline uint4 buf_ld128(Rsrc r, uint32_t boff)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, boff, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ inline void buf_st(Rsrc r, uint32_t boff, float v, float *)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, boff, 0, 0);
}
__device__ inline void buf_st(Rsrc r, uint32_t boff, float v, uint16_t *)
{
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)), r, boff, 0, 0);
}

// Loads / stores at a 32-bit byte offset from a wave-uniform base pointer.
template <class T>
__device__ inline T ld_at(const T *base, uint32_t boff)
{
    return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + boff);
}
__device__ inline void st_at(float *base, uint32_t boff, float v)
{
    *reinterpret_cast<float *>(reinterpret_cast<char *>(base) + boff) = v;
}
__device__ inline void st_at(uint16_t *base, uint32_t boff, float v)
{
    *reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(base) + boff) = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

__device__ inline float to_f32(float v) { return v; }
__device__ inline float to_f32(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(lo))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(hi))) << 16);
}

// ---------------------------------------------------------------- scalar maps
__device__ inline float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ inline float hw_log2(float v) { return __builtin_amdgcn_logf(v); }
__device__ inline float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// SiLU(v) = v * sigmoid(v) = v / (1 + e^-v).  For v -> -inf, 2^(+big) = inf and
// rcp(inf) = 0, so the result goes to -0 without NaN.
__device__ inline float silu(float v) { return v * hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

// softplus(a) * log2(e), accurate in relative terms for all a:
//   softplus(a) = max(a, 0) + log1p(e^-|a|).
// With e = 2^(-|a| log2 e) in (0, 1]: for e >= 1/32, log2(1 + e) is evaluated directly
// (1 + e >= 1.03, so rounding 1 + e costs < 2e-6 relative); below, the series
// log1p(e) = e (1 - e/2 + e^2/3 - e^3/4) has truncation error < e^4/5 < 2e-7 relative.
__device__ inline float softplus_log2(float a)
{
    const float a2 = a * kLog2e;
    const float e = hw_exp2(-__builtin_fabsf(a2));
    const float big = hw_log2(1.0f + e);
    float q = __builtin_fmaf(e, -0.25f, 0.33333333f);
    q = __builtin_fmaf(e, q, -0.5f);
    q = __builtin_fmaf(e, q, 1.0f);
    const float small = (e * kLog2e) * q;
    return __builtin_fmaxf(a2, 0.0f) + (e >= 0.03125f ? big : small);
}

}  // namespace samba
