// samba_scan.hip -- MI355X (gfx950) selective-scan core of a Mamba layer, C ABI.
//
// Operation (page "Samba: Simple Hybrid State Space Models for Efficient Unlimited
// Context Language Modeling", paper-graph-ui summary, section 3.4): causal depthwise
// conv (k = 4) + SiLU, Delta = softplus(dt + b), Abar = exp(Delta A),
// h_t = Abar h_{t-1} + Delta B_t u_t, y_t = C_t . h_t + D u_t, out = y * SiLU(z).
// Tap order, A = -exp(A_log) and the SiLU(z) gate as in "Samba Guide: Hybrid Mamba &
// Sliding Window Architecture", Step 1.
//
// This file holds the host entry points (argument checks, launch) and includes the
// kernels.  No CUDA, no compatibility layer: gfx950 only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>

#include "../../include/samba_scan.h"
#include "scan_common.h"
#include "scan_lane.h"
#include "scan_split.h"
#include "scan_decode.h"
#include "scan_conv.h"
#include "scan_bwd.h"
#include "scan_swa.h"
#include "scan_swa_decode.h"
#include "gemm.h"
#include "model_step.h"


namespace {

thread_local std::string g_err;

// Device memory of the allocation-free entry point (samba_swa_decode_noalloc): the split
// partials of the attention decode live in this file-scope array instead of a caller
// workspace.  Every GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device with hipGetSymbolAddress (scratch_on) and only that address
// is ever passed to a kernel.
constexpr size_t kNoAllocScratchBytes = size_t(24) << 20;  // 24 MiB
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call per
// device); nullptr, with the reason in g_err, when the lookup fails.
void *scratch_on(const char *fn)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        g_err = std::string(fn) + ": no usable current device: " + hipGetErrorString(e);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            g_err = std::string(fn) + ": hipGetSymbolAddress(scratch) failed: " + hipGetErrorString(e);
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

samba_status fail(samba_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
samba_status fail(samba_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

// Kernel choice for prefill / varlen.  The lane kernel (one lane per channel, 16 states
// in registers) is the cheapest per token when sequences x channels alone give at least
// two waves per SIMD (131072 lanes); otherwise the row kernels (16 lanes per channel) supply the
// parallelism: the two-role row kernel while the grid has at most one workgroup per CU,
// the single-role one (two workgroups per CU) beyond that.  SAMBA_SCAN_PATH=lane|single|
// split forces one of them (the tests run every kernel on every shape); the lane kernel is
// used whenever the row kernels' alignment requirement is not met.
enum class ScanPath { kLane, kSingle, kSplit };

ScanPath scan_path(int nseq, int d_inner, samba_dtype io)
{
    // The row kernels move 16-channel token rows as 16-byte vectors: every row must start
    // 16-byte aligned, i.e. d_inner * sizeof(element) must be a multiple of 16.
    const int elem = io == SAMBA_BF16 ? 2 : 4;
    if ((d_inner * elem) % 16 != 0) return ScanPath::kLane;
    const size_t row_grid = static_cast<size_t>(nseq) * static_cast<size_t>((d_inner + samba::rows::kChannels - 1) /
                                                                              samba::rows::kChannels);
    const ScanPath rows = row_grid <= static_cast<size_t>(samba::split::kMaxSplitGrid) ? ScanPath::kSplit
                                                                                       : ScanPath::kSingle;
    const char *e = getenv("SAMBA_SCAN_PATH");
    if (e != nullptr && e[0] != '\0') {
        if (strcmp(e, "lane") == 0) return ScanPath::kLane;
        if (strcmp(e, "single") == 0) return ScanPath::kSingle;
        if (strcmp(e, "split") == 0) return ScanPath::kSplit;
        if (strcmp(e, "rows") == 0) return rows;
    }
    constexpr size_t kLaneThreshold = 256ull * 4 * 64 * 2;  // lanes for 2 waves on each SIMD
    return static_cast<size_t>(nseq) * static_cast<size_t>(d_inner) < kLaneThreshold ? rows : ScanPath::kLane;
}

void launch_scan(const samba::ScanArgs &a, samba_dtype io, void *stream)
{
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (scan_path(a.nseq, a.D, io)) {
    case ScanPath::kLane: samba::launch_lane_scan(a, io, s); break;
    case ScanPath::kSingle: samba::launch_rows_single(a, io, s); break;
    case ScanPath::kSplit: samba::launch_rows_split(a, io, s); break;
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p, name)                                                               \
    do {                                                                                   \
        if ((p) == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: %s is NULL", fn, name); \
        if (!aligned16(p)) return fail(SAMBA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name); \
    } while (0)
#define OPTIONAL_PTR(p, name)                                                              \
    do {                                                                                   \
        if ((p) != nullptr && !aligned16(p))                                               \
            return fail(SAMBA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name); \
    } while (0)

samba_status check_common(const char *fn, int d_inner, int d_state, samba_dtype io,
                          const samba_params *p, bool needs_conv = true)
{
    if (d_inner < 1) return fail(SAMBA_ERR_INVALID_ARG, "%s: d_inner=%d must be >= 1", fn, d_inner);
    if (d_state < 1) return fail(SAMBA_ERR_INVALID_ARG, "%s: d_state=%d must be >= 1", fn, d_state);
    if (d_state > samba::kMaxState)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: d_state=%d exceeds the supported maximum %d", fn, d_state,
                    samba::kMaxState);
    if (io != SAMBA_F32 && io != SAMBA_BF16) return fail(SAMBA_ERR_INVALID_ARG, "%s: unknown io dtype %d", fn, (int)io);
    if (p == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: params is NULL", fn);
    REQUIRE_PTR(p->A, "params->A");
    if (needs_conv) REQUIRE_PTR(p->conv_w, "params->conv_w");
    OPTIONAL_PTR(p->D, "params->D");
    OPTIONAL_PTR(p->dt_bias, "params->dt_bias");
    OPTIONAL_PTR(p->conv_b, "params->conv_b");
    return SAMBA_OK;
}

samba_status launched(const char *fn)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SAMBA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    g_err.clear();
    return SAMBA_OK;
}

// Whether the byte ranges [p, p + pb) and [q, q + qb) share a byte.
bool overlaps(const void *p, size_t pb, const void *q, size_t qb)
{
    if (p == nullptr || q == nullptr || pb == 0 || qb == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + qb && b < a + pb;
}

// A named byte range of a call's arguments.
struct Span {
    const void *p;
    size_t bytes;
    const char *name;
};

// Fails (SAMBA_ERR_INVALID_ARG) when an output range shares a byte with an input range or with
// another output range.  Null pointers and empty ranges overlap nothing.
samba_status check_disjoint(const char *fn, std::initializer_list<Span> outs, std::initializer_list<Span> ins)
{
    for (const Span *o = outs.begin(); o != outs.end(); ++o) {
        for (const Span &i : ins)
            if (overlaps(o->p, o->bytes, i.p, i.bytes))
                return fail(SAMBA_ERR_INVALID_ARG, "%s: %s overlaps %s", fn, o->name, i.name);
        for (const Span *o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlaps(o->p, o->bytes, o2->p, o2->bytes))
                return fail(SAMBA_ERR_INVALID_ARG, "%s: %s overlaps %s", fn, o->name, o2->name);
    }
    return SAMBA_OK;
}

// Output / input disjointness of a prefill, varlen or backward call: token arrays of `tokens`
// rows, state and history arrays of `nseq` rows.
struct ScanSizes {
    size_t tok, bc, state, hist, vec, cw, a;
    ScanSizes(size_t tokens, int nseq, int d_inner, int d_state, samba_dtype io)
    {
        const size_t e = io == SAMBA_BF16 ? 2 : 4, D = static_cast<size_t>(d_inner), N = static_cast<size_t>(d_state);
        tok = tokens * D * e;
        bc = tokens * N * e;
        state = static_cast<size_t>(nseq) * D * N * 4;
        hist = static_cast<size_t>(nseq) * 3 * D * e;
        vec = D * 4;
        cw = D * samba::kConvK * 4;
        a = D * N * 4;
    }
};

// Builds the argument block shared by every kernel.

samba::ScanArgs make_args(int nseq, int seqlen, const int32_t *cu, int d_inner, int d_state,
                          const void *x, const void *dt, const void *B, const void *C, const void *z,
                          const samba_params *p, const float *h0, const void *conv0, void *out,
                          float *h_final, void *conv_final)
{
    samba::ScanArgs a{};
    a.nseq = nseq;
    a.seqlen = seqlen;
    a.cu = cu;
    a.total = 0;
    a.D = d_inner;
    a.N = d_state;
    a.x = x;
    a.dt = dt;
    a.B = B;
    a.C = C;
    a.z = z;
    a.A = p->A;
    a.Dskip = p->D;
    a.dt_bias = p->dt_bias;
    a.conv_w = p->conv_w;
    a.conv_b = p->conv_b;
    a.h0 = h0;
    a.conv0 = conv0;
    a.out = out;
    a.h_final = h_final;
    a.conv_final = conv_final;
    return a;
}

}  // namespace

extern "C" {

const char *samba_last_error(void) { return g_err.c_str(); }

const char *samba_version(void) { return "samba_scan 0.1 (gfx950)"; }

size_t samba_scan_workspace_bytes(int nseq, int max_seqlen, int d_inner, int d_state)
{
    (void)nseq;
    (void)max_seqlen;
    (void)d_inner;
    (void)d_state;
    return 0;
}

}  // extern "C"

namespace {

// Outputs of a prefill / varlen call (out, h_final, conv_final) against its inputs and each
// other.  h_final may be h0 itself and conv_final conv0 itself (the state updated in place:
// every channel's state and history are read before they are written, by the same threads
// or across a workgroup barrier); any other overlap is refused.
samba_status scan_disjoint(const char *fn, bool u_in, size_t tokens, int nseq, int d_inner, int d_state,
                           samba_dtype io, const int32_t *cu, const void *x, const void *dt, const void *B,
                           const void *C, const void *z, const samba_params *p, const float *h0, const void *conv0,
                           const void *out, const float *h_final, const void *conv_final)
{
    const ScanSizes n(tokens, nseq, d_inner, d_state, io);
    const size_t hist = u_in ? 0 : n.hist;
    return check_disjoint(fn, {{out, n.tok, "out"}, {h_final, n.state, "h_final"}, {conv_final, hist, "conv_final"}},
                          {{x, n.tok, u_in ? "u" : "x"}, {dt, n.tok, "dt"}, {z, n.tok, "z"}, {B, n.bc, "B"},
                           {C, n.bc, "C"}, {h0 == h_final ? nullptr : h0, n.state, "h0"},
                           {conv0 == conv_final ? nullptr : conv0, hist, "conv0"},
                           {cu, cu != nullptr ? (static_cast<size_t>(nseq) + 1) * 4 : 0, "cu_seqlens"},
                           {p->A, n.a, "params->A"}, {p->D, n.vec, "params->D"}, {p->dt_bias, n.vec, "params->dt_bias"},
                           {u_in ? nullptr : p->conv_w, n.cw, "params->conv_w"},
                           {u_in ? nullptr : p->conv_b, n.vec, "params->conv_b"}});
}

// Fixed-length prefill, x (pre-conv) or u (u_in) as the token input.
samba_status prefill_impl(const char *fn, bool u_in, int batch, int seqlen, int d_inner, int d_state, samba_dtype io,
                          const void *x, const void *dt, const void *B, const void *C, const void *z,
                          const samba_params *params, const float *h0, const void *conv0, void *out, float *h_final,
                          void *conv_final, void *stream)
{
    if (batch < 0 || seqlen < 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: batch=%d seqlen=%d must be >= 0", fn, batch, seqlen);
    samba_status st = check_common(fn, d_inner, d_state, io, params, !u_in);
    if (st != SAMBA_OK) return st;
    if (batch == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    if ((size_t)batch * (size_t)seqlen > (size_t)INT32_MAX)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: batch*seqlen=%zu exceeds 2^31-1 tokens", fn,
                    (size_t)batch * (size_t)seqlen);
    if (seqlen > 0) {
        REQUIRE_PTR(x, u_in ? "u" : "x");
        REQUIRE_PTR(dt, "dt");
        REQUIRE_PTR(B, "B");
        REQUIRE_PTR(C, "C");
        REQUIRE_PTR(out, "out");
        OPTIONAL_PTR(z, "z");
    }
    OPTIONAL_PTR(h0, "h0");
    OPTIONAL_PTR(conv0, "conv0");
    OPTIONAL_PTR(h_final, "h_final");
    OPTIONAL_PTR(conv_final, "conv_final");
    st = scan_disjoint(fn, u_in, static_cast<size_t>(batch) * static_cast<size_t>(seqlen), batch, d_inner, d_state, io,
                       nullptr, x, dt, B, C, z, params, h0, conv0, out, h_final, conv_final);
    if (st != SAMBA_OK) return st;
    samba::ScanArgs a = make_args(batch, seqlen, nullptr, d_inner, d_state, x, dt, B, C, z, params, h0,
                                  conv0, out, h_final, conv_final);
    a.u_in = u_in;
    launch_scan(a, io, stream);
    return launched(fn);
}

// Packed variable-length prefill, x (pre-conv) or u (u_in) as the token input.
samba_status varlen_impl(const char *fn, bool u_in, int nseq, const int32_t *cu_seqlens, int total_tokens,
                         int max_seqlen, int d_inner, int d_state, samba_dtype io, const void *x, const void *dt,
                         const void *B, const void *C, const void *z, const samba_params *params, const float *h0,
                         const void *conv0, void *out, float *h_final, void *conv_final, void *stream)
{
    if (nseq < 0 || total_tokens < 0 || max_seqlen < 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: nseq=%d total_tokens=%d max_seqlen=%d must be >= 0", fn, nseq,
                    total_tokens, max_seqlen);
    samba_status st = check_common(fn, d_inner, d_state, io, params, !u_in);
    if (st != SAMBA_OK) return st;
    if (nseq == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    if (cu_seqlens == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: cu_seqlens is NULL", fn);
    if (max_seqlen > total_tokens)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: max_seqlen=%d exceeds total_tokens=%d", fn, max_seqlen, total_tokens);
    if (total_tokens > 0) {
        REQUIRE_PTR(x, u_in ? "u" : "x");
        REQUIRE_PTR(dt, "dt");
        REQUIRE_PTR(B, "B");
        REQUIRE_PTR(C, "C");
        REQUIRE_PTR(out, "out");
        OPTIONAL_PTR(z, "z");
    }
    OPTIONAL_PTR(h0, "h0");
    OPTIONAL_PTR(conv0, "conv0");
    OPTIONAL_PTR(h_final, "h_final");
    OPTIONAL_PTR(conv_final, "conv_final");
    st = scan_disjoint(fn, u_in, static_cast<size_t>(total_tokens), nseq, d_inner, d_state, io, cu_seqlens, x, dt, B, C,
                       z, params, h0, conv0, out, h_final, conv_final);
    if (st != SAMBA_OK) return st;
    samba::ScanArgs a = make_args(nseq, max_seqlen, cu_seqlens, d_inner, d_state, x, dt, B, C, z, params, h0,
                                  conv0, out, h_final, conv_final);
    a.total = total_tokens;
    a.u_in = u_in;
    launch_scan(a, io, stream);
    return launched(fn);
}

}  // namespace

extern "C" {

samba_status samba_scan_prefill(int batch, int seqlen, int d_inner, int d_state, samba_dtype io,
                                const void *x, const void *dt, const void *B, const void *C,
                                const void *z, const samba_params *params,
                                const float *h0, const void *conv0,
                                void *out, float *h_final, void *conv_final,
                                void *workspace, size_t workspace_bytes, void *stream)
{
    (void)workspace;
    (void)workspace_bytes;
    return prefill_impl("samba_scan_prefill", false, batch, seqlen, d_inner, d_state, io, x, dt, B, C, z, params, h0,
                        conv0, out, h_final, conv_final, stream);
}

samba_status samba_scan_prefill_u(int batch, int seqlen, int d_inner, int d_state, samba_dtype io,
                                  const void *u, const void *dt, const void *B, const void *C,
                                  const void *z, const samba_params *params, const float *h0,
                                  void *out, float *h_final, void *workspace, size_t workspace_bytes, void *stream)
{
    (void)workspace;
    (void)workspace_bytes;
    return prefill_impl("samba_scan_prefill_u", true, batch, seqlen, d_inner, d_state, io, u, dt, B, C, z, params, h0,
                        nullptr, out, h_final, nullptr, stream);
}

samba_status samba_scan_varlen(int nseq, const int32_t *cu_seqlens, int total_tokens, int max_seqlen,
                               int d_inner, int d_state, samba_dtype io,
                               const void *x, const void *dt, const void *B, const void *C,
                               const void *z, const samba_params *params,
                               const float *h0, const void *conv0,
                               void *out, float *h_final, void *conv_final,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    (void)workspace;
    (void)workspace_bytes;
    return varlen_impl("samba_scan_varlen", false, nseq, cu_seqlens, total_tokens, max_seqlen, d_inner, d_state, io, x,
                       dt, B, C, z, params, h0, conv0, out, h_final, conv_final, stream);
}

samba_status samba_scan_varlen_u(int nseq, const int32_t *cu_seqlens, int total_tokens, int max_seqlen,
                                 int d_inner, int d_state, samba_dtype io, const void *u, const void *dt,
                                 const void *B, const void *C, const void *z, const samba_params *params,
                                 const float *h0, void *out, float *h_final, void *workspace,
                                 size_t workspace_bytes, void *stream)
{
    (void)workspace;
    (void)workspace_bytes;
    return varlen_impl("samba_scan_varlen_u", true, nseq, cu_seqlens, total_tokens, max_seqlen, d_inner, d_state, io,
                       u, dt, B, C, z, params, h0, nullptr, out, h_final, nullptr, stream);
}

samba_status samba_scan_decode(int nseq, int d_inner, int d_state, samba_dtype io,
                               const void *x, const void *dt, const void *B, const void *C,
                               const void *z, const samba_params *params,
                               float *h, void *conv_ring, const int32_t *ring_head_in, int32_t *ring_head_out,
                               void *out, void *stream)
{
    const char *fn = "samba_scan_decode";
    if (nseq < 0) return fail(SAMBA_ERR_INVALID_ARG, "%s: nseq=%d must be >= 0", fn, nseq);
    samba_status st = check_common(fn, d_inner, d_state, io, params);
    if (st != SAMBA_OK) return st;
    if (nseq == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    // one grid row per sequence
    if (nseq > 65535) return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq=%d exceeds 65535", fn, nseq);
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(dt, "dt");
    REQUIRE_PTR(B, "B");
    REQUIRE_PTR(C, "C");
    REQUIRE_PTR(out, "out");
    REQUIRE_PTR(h, "h");
    REQUIRE_PTR(conv_ring, "conv_ring");
    if (ring_head_in == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: ring_head_in is NULL", fn);
    if ((reinterpret_cast<uintptr_t>(ring_head_in) & 3u) != 0 || (reinterpret_cast<uintptr_t>(ring_head_out) & 3u) != 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: ring heads must be 4-byte aligned", fn);
    const size_t head_bytes = static_cast<size_t>(nseq) * sizeof(int32_t);
    if (overlaps(ring_head_out, head_bytes, ring_head_in, head_bytes))
        return fail(SAMBA_ERR_INVALID_ARG, "%s: ring_head_out overlaps ring_head_in (the heads are double-buffered: "
                    "every workgroup of a sequence reads its head)", fn);
    OPTIONAL_PTR(z, "z");
    {
        // h and the conv ring are read and written in place: they may not overlap anything else.
        const ScanSizes n(static_cast<size_t>(nseq), nseq, d_inner, d_state, io);
        st = check_disjoint(fn, {{out, n.tok, "out"}, {h, n.state, "h"}, {conv_ring, n.hist, "conv_ring"},
                                 {ring_head_out, head_bytes, "ring_head_out"}},
                            {{x, n.tok, "x"}, {dt, n.tok, "dt"}, {z, n.tok, "z"}, {B, n.bc, "B"}, {C, n.bc, "C"},
                             {ring_head_in, head_bytes, "ring_head_in"}, {params->A, n.a, "params->A"},
                             {params->D, n.vec, "params->D"}, {params->dt_bias, n.vec, "params->dt_bias"},
                             {params->conv_w, n.cw, "params->conv_w"}, {params->conv_b, n.vec, "params->conv_b"}});
        if (st != SAMBA_OK) return st;
    }
    // A decode step is the recurrence over a single token whose state and history are
    // read and written in place.
    samba::ScanArgs a = make_args(nseq, 1, nullptr, d_inner, d_state, x, dt, B, C, z, params, h, conv_ring,
                                  out, h, conv_ring);
    a.head_in = ring_head_in;
    a.head_out = ring_head_out;
    if (d_state == samba::kMaxState)
        samba::launch_decode16(a, io, static_cast<hipStream_t>(stream));
    else
        samba::launch_lane_scan(a, io, static_cast<hipStream_t>(stream));
    return launched(fn);
}

samba_status samba_conv_silu(int nseq, const int32_t *cu_seqlens, int seqlen, int total_tokens, int d_inner,
                             samba_dtype io, const void *x, const float *conv_w, const float *conv_b,
                             const void *conv0, void *u, void *conv_final, void *stream)
{
    const char *fn = "samba_conv_silu";
    if (nseq < 0 || seqlen < 0 || (cu_seqlens != nullptr && total_tokens < 0))
        return fail(SAMBA_ERR_INVALID_ARG, "%s: nseq=%d seqlen=%d total_tokens=%d must be >= 0", fn, nseq, seqlen,
                    total_tokens);
    if (d_inner < 1) return fail(SAMBA_ERR_INVALID_ARG, "%s: d_inner=%d must be >= 1", fn, d_inner);
    if (io != SAMBA_F32 && io != SAMBA_BF16) return fail(SAMBA_ERR_INVALID_ARG, "%s: unknown io dtype %d", fn, (int)io);
    if (nseq == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    const size_t elem = io == SAMBA_BF16 ? 2 : 4;
    size_t tokens;
    if (cu_seqlens != nullptr) {
        if (seqlen > total_tokens)
            return fail(SAMBA_ERR_INVALID_ARG, "%s: max_seqlen=%d exceeds total_tokens=%d", fn, seqlen, total_tokens);
        tokens = static_cast<size_t>(total_tokens);
    } else {
        tokens = static_cast<size_t>(nseq) * static_cast<size_t>(seqlen);
        if (tokens > static_cast<size_t>(INT32_MAX))
            return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq*seqlen=%zu exceeds 2^31-1 tokens", fn, tokens);
    }
    REQUIRE_PTR(conv_w, "conv_w");
    OPTIONAL_PTR(conv_b, "conv_b");
    if (tokens > 0) {
        REQUIRE_PTR(x, "x");
        REQUIRE_PTR(u, "u");
    }
    OPTIONAL_PTR(conv0, "conv0");
    OPTIONAL_PTR(conv_final, "conv_final");
    const size_t tok_bytes = tokens * static_cast<size_t>(d_inner) * elem;
    const size_t hist_bytes = static_cast<size_t>(nseq) * 3 * static_cast<size_t>(d_inner) * elem;
    if (overlaps(u, tok_bytes, x, tok_bytes))
        return fail(SAMBA_ERR_INVALID_ARG, "%s: u overlaps x (runs of tokens re-read the rows before them)", fn);
    if (overlaps(conv_final, hist_bytes, conv0, hist_bytes))
        return fail(SAMBA_ERR_INVALID_ARG, "%s: conv_final overlaps conv0", fn);
    const long long run = std::max<long long>(samba::conv::kMinRun, (static_cast<long long>(seqlen) + 65534) / 65535);
    const long long nruns = std::max<long long>(1, (seqlen + run - 1) / run);
    if (static_cast<long long>(nseq) * nruns > INT32_MAX)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq=%d x %lld runs exceeds the launch limit", fn, nseq, nruns);
    samba::ConvArgs a{};
    a.nseq = nseq;
    a.seqlen = seqlen;
    a.cu = cu_seqlens;
    a.total = total_tokens;
    a.D = d_inner;
    a.x = x;
    a.conv_w = conv_w;
    a.conv_b = conv_b;
    a.conv0 = conv0;
    a.u = u;
    a.conv_final = conv_final;
    samba::launch_conv_silu(a, io, static_cast<hipStream_t>(stream));
    return launched(fn);
}

size_t samba_scan_backward_workspace_bytes(int nseq, int seqlen, int total_tokens, int d_inner, int d_state)
{
    (void)d_state;
    if (nseq <= 0 || seqlen < 0 || total_tokens < 0 || d_inner <= 0) return 0;
    return samba::bwd_workspace(nseq, seqlen, total_tokens, d_inner).total_bytes;
}

samba_status samba_scan_backward(int nseq, const int32_t *cu_seqlens, int seqlen, int total_tokens, int d_inner,
                                 int d_state, samba_dtype io, const void *x, const void *dt, const void *B,
                                 const void *C, const void *z, const samba_params *params, const float *h0,
                                 const void *conv0, const void *dout, const float *dh_final,
                                 const void *dconv_final, void *dx, void *ddt, void *dB, void *dC, void *dz,
                                 float *dA, float *dD, float *ddt_bias, float *dconv_w, float *dconv_b,
                                 float *dh0, void *dconv0, void *workspace, size_t workspace_bytes, void *stream)
{
    const char *fn = "samba_scan_backward";
    if (nseq < 0 || seqlen < 0 || (cu_seqlens != nullptr && total_tokens < 0))
        return fail(SAMBA_ERR_INVALID_ARG, "%s: nseq=%d seqlen=%d total_tokens=%d must be >= 0", fn, nseq, seqlen,
                    total_tokens);
    samba_status st = check_common(fn, d_inner, d_state, io, params);
    if (st != SAMBA_OK) return st;
    if (nseq == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    size_t tokens;
    if (cu_seqlens != nullptr) {
        if (seqlen > total_tokens)
            return fail(SAMBA_ERR_INVALID_ARG, "%s: max_seqlen=%d exceeds total_tokens=%d", fn, seqlen, total_tokens);
        tokens = static_cast<size_t>(total_tokens);
    } else {
        tokens = static_cast<size_t>(nseq) * static_cast<size_t>(seqlen);
        if (tokens > static_cast<size_t>(INT32_MAX))
            return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq*seqlen=%zu exceeds 2^31-1 tokens", fn, tokens);
    }
    if (nseq > 65535 || (seqlen + samba::bwd::kChunk - 1) / samba::bwd::kChunk > 65535)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq=%d or seqlen=%d exceeds the launch limits (65535 sequences, "
                    "65535 chunks of %d tokens)", fn, nseq, seqlen, samba::bwd::kChunk);
    if (tokens > 0) {
        REQUIRE_PTR(x, "x");
        REQUIRE_PTR(dt, "dt");
        REQUIRE_PTR(B, "B");
        REQUIRE_PTR(C, "C");
        REQUIRE_PTR(dout, "dout");
        REQUIRE_PTR(dx, "dx");
        REQUIRE_PTR(ddt, "ddt");
        REQUIRE_PTR(dB, "dB");
        REQUIRE_PTR(dC, "dC");
        OPTIONAL_PTR(z, "z");
        if (z != nullptr) REQUIRE_PTR(dz, "dz");
    }
    REQUIRE_PTR(dA, "dA");
    REQUIRE_PTR(dD, "dD");
    REQUIRE_PTR(ddt_bias, "ddt_bias");
    REQUIRE_PTR(dconv_w, "dconv_w");
    REQUIRE_PTR(dconv_b, "dconv_b");
    OPTIONAL_PTR(h0, "h0");
    OPTIONAL_PTR(conv0, "conv0");
    OPTIONAL_PTR(dh_final, "dh_final");
    OPTIONAL_PTR(dconv_final, "dconv_final");
    OPTIONAL_PTR(dh0, "dh0");
    OPTIONAL_PTR(dconv0, "dconv0");
    const size_t need = samba::bwd_workspace(nseq, seqlen, static_cast<int>(tokens), d_inner).total_bytes;
    if (workspace == nullptr || workspace_bytes < need)
        return fail(SAMBA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace == nullptr ? (size_t)0 : workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
    {
        const ScanSizes n(tokens, nseq, d_inner, d_state, io);
        st = check_disjoint(
            fn,
            {{dx, n.tok, "dx"}, {ddt, n.tok, "ddt"}, {dz, z != nullptr ? n.tok : 0, "dz"}, {dB, n.bc, "dB"},
             {dC, n.bc, "dC"}, {dA, n.a, "dA"}, {dD, n.vec, "dD"}, {ddt_bias, n.vec, "ddt_bias"},
             {dconv_w, n.cw, "dconv_w"}, {dconv_b, n.vec, "dconv_b"}, {dh0, n.state, "dh0"},
             {dconv0, n.hist, "dconv0"}, {workspace, need, "workspace"}},
            {{x, n.tok, "x"}, {dt, n.tok, "dt"}, {z, n.tok, "z"}, {dout, n.tok, "dout"}, {B, n.bc, "B"},
             {C, n.bc, "C"}, {h0, n.state, "h0"}, {dh_final, n.state, "dh_final"}, {conv0, n.hist, "conv0"},
             {dconv_final, n.hist, "dconv_final"},
             {cu_seqlens, cu_seqlens != nullptr ? (static_cast<size_t>(nseq) + 1) * 4 : 0, "cu_seqlens"},
             {params->A, n.a, "params->A"}, {params->D, n.vec, "params->D"},
             {params->dt_bias, n.vec, "params->dt_bias"}, {params->conv_w, n.cw, "params->conv_w"},
             {params->conv_b, n.vec, "params->conv_b"}});
        if (st != SAMBA_OK) return st;
    }
    samba::BwdArgs a{};
    a.nseq = nseq;
    a.seqlen = seqlen;
    a.cu = cu_seqlens;
    a.total = static_cast<int>(tokens);
    a.D = d_inner;
    a.N = d_state;
    a.x = x;
    a.dt = dt;
    a.B = B;
    a.C = C;
    a.z = z;
    a.A = params->A;
    a.Dskip = params->D;
    a.dt_bias = params->dt_bias;
    a.conv_w = params->conv_w;
    a.conv_b = params->conv_b;
    a.h0 = h0;
    a.conv0 = conv0;
    a.dout = dout;
    a.dh_final = dh_final;
    a.dconv_final = dconv_final;
    a.dx = dx;
    a.ddt = ddt;
    a.dB = dB;
    a.dC = dC;
    a.dz = dz;
    a.dA = dA;
    a.dD = dD;
    a.ddt_bias = ddt_bias;
    a.dconv_w = dconv_w;
    a.dconv_b = dconv_b;
    a.dh0 = dh0;
    a.dconv0 = dconv0;
    samba::launch_backward(a, static_cast<float *>(workspace), io, static_cast<hipStream_t>(stream));
    return launched(fn);
}

size_t samba_swa_workspace_bytes(int total_tokens, int n_kv_heads, int head_dim)
{
    if (total_tokens <= 0 || n_kv_heads <= 0 || head_dim <= 0) return 0;
    return samba::swa_workspace_bytes(total_tokens, n_kv_heads, head_dim);
}

samba_status samba_swa_prefill(int nseq, const int32_t *cu_seqlens, int seqlen, int total_tokens, int n_heads,
                               int n_kv_heads, int head_dim, int window, float rope_base, samba_dtype io,
                               const void *q, const void *k, const void *v, void *out, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    const char *fn = "samba_swa_prefill";
    if (nseq < 0 || seqlen < 0 || (cu_seqlens != nullptr && total_tokens < 0) || window < 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: nseq=%d seqlen=%d total_tokens=%d window=%d must be >= 0", fn, nseq,
                    seqlen, total_tokens, window);
    if (io != SAMBA_BF16)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: io dtype %d: attention takes bfloat16 (the matrix-core operand type)",
                    fn, (int)io);
    if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads != 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: n_heads=%d must be a positive multiple of n_kv_heads=%d", fn, n_heads,
                    n_kv_heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: head_dim=%d (64 and 128 are built)", fn, head_dim);
    if (!(rope_base > 1.0f)) return fail(SAMBA_ERR_INVALID_ARG, "%s: rope_base must be > 1", fn);
    if (nseq == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    size_t tokens;
    if (cu_seqlens != nullptr) {
        if (seqlen > total_tokens)
            return fail(SAMBA_ERR_INVALID_ARG, "%s: max_seqlen=%d exceeds total_tokens=%d", fn, seqlen, total_tokens);
        tokens = static_cast<size_t>(total_tokens);
    } else {
        tokens = static_cast<size_t>(nseq) * static_cast<size_t>(seqlen);
        if (tokens > static_cast<size_t>(INT32_MAX))
            return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq*seqlen=%zu exceeds 2^31-1 tokens", fn, tokens);
    }
    if (static_cast<double>(nseq) * n_heads * ((seqlen + 63) / 64) > 2147483647.0)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq x n_heads x row blocks exceeds 2^31-1 workgroups", fn);
    if (tokens == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    REQUIRE_PTR(q, "q");
    REQUIRE_PTR(k, "k");
    REQUIRE_PTR(v, "v");
    REQUIRE_PTR(out, "out");
    const size_t need = samba::swa_workspace_bytes(static_cast<int>(tokens), n_kv_heads, head_dim);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(SAMBA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace == nullptr ? (size_t)0 : workspace_bytes);
    REQUIRE_PTR(workspace, "workspace");
    {
        const size_t qo = tokens * n_heads * head_dim * 2, kv = tokens * n_kv_heads * head_dim * 2;
        samba_status st = check_disjoint(
            fn, {{out, qo, "out"}, {workspace, need, "workspace"}},
            {{q, qo, "q"}, {k, kv, "k"}, {v, kv, "v"},
             {cu_seqlens, cu_seqlens != nullptr ? (static_cast<size_t>(nseq) + 1) * 4 : 0, "cu_seqlens"}});
        if (st != SAMBA_OK) return st;
    }
    samba::SwaArgs a{};
    a.nseq = nseq;
    a.seqlen = seqlen;
    a.cu = cu_seqlens;
    a.total = static_cast<int>(tokens);
    a.Hq = n_heads;
    a.Hkv = n_kv_heads;
    a.dh = head_dim;
    a.window = window;
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(head_dim)));
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.krot = static_cast<uint16_t *>(workspace);
    samba::swa_set_theta(a, static_cast<double>(rope_base));
    samba::launch_swa(a, static_cast<hipStream_t>(stream));
    return launched(fn);
}

size_t samba_swa_decode_workspace_bytes(int nseq, int n_heads, int head_dim)
{
    if (nseq <= 0 || n_heads <= 0 || head_dim <= 0) return 0;
    return samba::swa_decode_workspace_bytes(nseq, n_heads, head_dim);
}

namespace {
samba::SwaDecArgs swa_dec_args(int nseq, int n_heads, int n_kv_heads, int head_dim, int window, float rope_base,
                               const void *q, const void *k, const void *v, const int32_t *pos, void *k_cache,
                               void *v_cache, void *out, void *workspace)
{
    samba::SwaDecArgs a{};
    a.S = nseq;
    a.Hq = n_heads;
    a.Hkv = n_kv_heads;
    a.dh = head_dim;
    a.window = window;
    a.cap = window + 1;
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(head_dim)));
    a.q = q;
    a.k = k;
    a.v = v;
    a.pos = pos;
    a.kc = static_cast<uint16_t *>(k_cache);
    a.vc = static_cast<uint16_t *>(v_cache);
    a.out = out;
    a.part = static_cast<float *>(workspace);
    samba::swa_dec_set_theta(a, static_cast<double>(rope_base));
    return a;
}

samba_status swa_dec_common(const char *fn, int nseq, int n_heads, int n_kv_heads, int head_dim, int window,
                            float rope_base, samba_dtype io, bool decode)
{
    if (nseq < 0 || window < 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: nseq=%d window=%d must be >= 0", fn, nseq, window);
    if (io != SAMBA_BF16)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: io dtype %d: attention takes bfloat16", fn, (int)io);
    if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads != 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: n_heads=%d must be a positive multiple of n_kv_heads=%d", fn, n_heads,
                    n_kv_heads);
    if (decode && n_heads / n_kv_heads > samba::swadec::kMaxGroup)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: %d query heads per KV head (at most %d are built)", fn,
                    n_heads / n_kv_heads, samba::swadec::kMaxGroup);
    if (head_dim != 64 && head_dim != 128)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: head_dim=%d (64 and 128 are built)", fn, head_dim);
    if (!(rope_base > 1.0f)) return fail(SAMBA_ERR_INVALID_ARG, "%s: rope_base must be > 1", fn);
    if (window >= 65535 * 64)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: window=%d exceeds the launch limit", fn, window);
    if (nseq > 65535) return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq=%d exceeds 65535", fn, nseq);
    return SAMBA_OK;
}

// Outputs of an attention decode step (out, both rings, the partials) against its inputs and
// each other; rings are [nseq][n_kv_heads][window + 1][head_dim] bf16.
samba_status swa_dec_disjoint(const char *fn, int nseq, int n_heads, int n_kv_heads, int head_dim, int window,
                              const void *q, const void *k, const void *v, const int32_t *pos, const void *k_cache,
                              const void *v_cache, const void *out, const void *workspace, size_t ws_bytes)
{
    const size_t S = static_cast<size_t>(nseq), dh = static_cast<size_t>(head_dim);
    const size_t qo = S * n_heads * dh * 2, kv = S * n_kv_heads * dh * 2;
    const size_t ring = S * n_kv_heads * (static_cast<size_t>(window) + 1) * dh * 2;
    return check_disjoint(fn,
                          {{out, qo, "out"}, {k_cache, ring, "k_cache"}, {v_cache, ring, "v_cache"},
                           {workspace, ws_bytes, "workspace"}},
                          {{q, qo, "q"}, {k, kv, "k"}, {v, kv, "v"}, {pos, S * 4, "pos"}});
}
}  // namespace

samba_status samba_swa_decode(int nseq, int n_heads, int n_kv_heads, int head_dim, int window, float rope_base,
                              samba_dtype io, const void *q, const void *k, const void *v, const int32_t *pos,
                              void *k_cache, void *v_cache, void *out, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    const char *fn = "samba_swa_decode";
    samba_status st = swa_dec_common(fn, nseq, n_heads, n_kv_heads, head_dim, window, rope_base, io, true);
    if (st != SAMBA_OK) return st;
    if (nseq == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    REQUIRE_PTR(q, "q");
    REQUIRE_PTR(k, "k");
    REQUIRE_PTR(v, "v");
    REQUIRE_PTR(out, "out");
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    if (pos == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: pos is NULL", fn);
    const size_t need = samba::swa_decode_workspace_bytes(nseq, n_heads, head_dim);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(SAMBA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace == nullptr ? (size_t)0 : workspace_bytes);
    REQUIRE_PTR(workspace, "workspace");
    st = swa_dec_disjoint(fn, nseq, n_heads, n_kv_heads, head_dim, window, q, k, v, pos, k_cache, v_cache, out,
                          workspace, need);
    if (st != SAMBA_OK) return st;
    samba::SwaDecArgs a = swa_dec_args(nseq, n_heads, n_kv_heads, head_dim, window, rope_base, q, k, v, pos, k_cache,
                                       v_cache, out, workspace);
    samba::launch_swa_decode(a, static_cast<hipStream_t>(stream));
    return launched(fn);
}

size_t samba_swa_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

samba_status samba_swa_decode_noalloc(int nseq, int n_heads, int n_kv_heads, int head_dim, int window, float rope_base,
                                      samba_dtype io, const void *q, const void *k, const void *v, const int32_t *pos,
                                      void *k_cache, void *v_cache, void *out, void *stream)
{
    const char *fn = "samba_swa_decode_noalloc";
    samba_status st = swa_dec_common(fn, nseq, n_heads, n_kv_heads, head_dim, window, rope_base, io, true);
    if (st != SAMBA_OK) return st;
    if (nseq == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    const size_t need = samba::swa_decode_workspace_bytes(nseq, n_heads, head_dim);
    if (need > kNoAllocScratchBytes)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq=%d x n_heads=%d x head_dim=%d needs %zu bytes of split partials, "
                    "more than the %zu bytes of the library's scratch array (use samba_swa_decode with a "
                    "workspace)", fn, nseq, n_heads, head_dim, need, kNoAllocScratchBytes);
    REQUIRE_PTR(q, "q");
    REQUIRE_PTR(k, "k");
    REQUIRE_PTR(v, "v");
    REQUIRE_PTR(out, "out");
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    if (pos == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: pos is NULL", fn);
    st = swa_dec_disjoint(fn, nseq, n_heads, n_kv_heads, head_dim, window, q, k, v, pos, k_cache, v_cache, out,
                          nullptr, 0);
    if (st != SAMBA_OK) return st;
    void *part = scratch_on(fn);
    if (part == nullptr) return SAMBA_ERR_HIP;
    // Every partial the combine reads is written by the attention kernel of the same call
    // (inactive sequences included), so the array needs no clearing.
    samba::SwaDecArgs a = swa_dec_args(nseq, n_heads, n_kv_heads, head_dim, window, rope_base, q, k, v, pos, k_cache,
                                       v_cache, out, part);
    samba::launch_swa_decode(a, static_cast<hipStream_t>(stream));
    return launched(fn);
}

samba_status samba_swa_kv_fill(int nseq, const int32_t *cu_seqlens, int seqlen, int total_tokens, int n_kv_heads,
                               int head_dim, int window, float rope_base, samba_dtype io, const void *k,
                               const void *v, void *k_cache, void *v_cache, void *stream)
{
    const char *fn = "samba_swa_kv_fill";
    samba_status st = swa_dec_common(fn, nseq, n_kv_heads, n_kv_heads, head_dim, window, rope_base, io, false);
    if (st != SAMBA_OK) return st;
    if (seqlen < 0 || (cu_seqlens != nullptr && total_tokens < 0))
        return fail(SAMBA_ERR_INVALID_ARG, "%s: seqlen=%d total_tokens=%d must be >= 0", fn, seqlen, total_tokens);
    if (nseq == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    size_t tokens = cu_seqlens != nullptr ? static_cast<size_t>(total_tokens)
                                          : static_cast<size_t>(nseq) * static_cast<size_t>(seqlen);
    if (tokens > static_cast<size_t>(INT32_MAX))
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: %zu tokens exceed 2^31-1", fn, tokens);
    if (tokens > 0) {
        REQUIRE_PTR(k, "k");
        REQUIRE_PTR(v, "v");
    }
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    {
        const size_t kv = tokens * n_kv_heads * static_cast<size_t>(head_dim) * 2;
        const size_t ring = static_cast<size_t>(nseq) * n_kv_heads * (static_cast<size_t>(window) + 1) * head_dim * 2;
        st = check_disjoint(fn, {{k_cache, ring, "k_cache"}, {v_cache, ring, "v_cache"}},
                            {{k, kv, "k"}, {v, kv, "v"},
                             {cu_seqlens, cu_seqlens != nullptr ? (static_cast<size_t>(nseq) + 1) * 4 : 0,
                              "cu_seqlens"}});
        if (st != SAMBA_OK) return st;
    }
    samba::SwaDecArgs a{};
    a.S = nseq;
    a.Hq = n_kv_heads;
    a.Hkv = n_kv_heads;
    a.dh = head_dim;
    a.window = window;
    a.cap = window + 1;
    a.k = k;
    a.v = v;
    a.kc = static_cast<uint16_t *>(k_cache);
    a.vc = static_cast<uint16_t *>(v_cache);
    a.cu = cu_seqlens;
    a.seqlen = seqlen;
    a.total = static_cast<int>(tokens);
    samba::swa_dec_set_theta(a, static_cast<double>(rope_base));
    samba::launch_swa_kv_fill(a, static_cast<hipStream_t>(stream));
    return launched(fn);
}

size_t samba_gemm_workspace_bytes(int M, int N, int K, samba_gemm_epilogue epilogue)
{
    if (M <= 0 || N <= 0 || K <= 0 || epilogue < SAMBA_GEMM_STORE || epilogue > SAMBA_GEMM_SWIGLU) return 0;
    return samba::gemm::plan(M, N, K, static_cast<int>(epilogue)).part_bytes;
}

namespace {
// Work the split-K reduce of a decode-step projection can do on the way (see
// samba::gemm::norm_fusable / conv_fusable); the flags tell the caller what was done.
struct GemmFuse {
    const float *norm_w = nullptr;  // add: RMSNorm of the new rows into norm_out
    float norm_eps = 0.f;
    uint16_t *norm_out = nullptr;
    const float *conv_w = nullptr, *conv_b = nullptr;  // store: u = SiLU(conv(x)) of the x half
    const uint16_t *conv0 = nullptr;
    const int32_t *conv_head = nullptr;  // conv0 is a ring with these heads (nullptr: oldest first)
    uint16_t *conv_u = nullptr;
    int conv_D = 0;
    bool normed = false, conved = false;
};

// samba_gemm, optionally with the work of a GemmFuse done by its split-K reduce.
samba_status gemm_impl(int M, int N, int K, samba_gemm_epilogue epilogue, const void *A, int lda, const void *W,
                       void *out, int ldo, const float *residual, int ldr, void *workspace, size_t workspace_bytes,
                       void *stream, GemmFuse *fz = nullptr)
{
    if (fz != nullptr) fz->normed = fz->conved = false;
    const char *fn = "samba_gemm";
    if (M < 0 || N < 0 || K < 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: M=%d N=%d K=%d must be >= 0", fn, M, N, K);
    if (epilogue < SAMBA_GEMM_STORE || epilogue > SAMBA_GEMM_SWIGLU)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: unknown epilogue %d", fn, (int)epilogue);
    if (K % 8 != 0) return fail(SAMBA_ERR_UNSUPPORTED, "%s: K=%d is not a multiple of 8", fn, K);
    if (M == 0 || N == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    if (lda < K || lda % 8 != 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: lda=%d must be >= K=%d and a multiple of 8", fn, lda, K);
    if (ldo < N) return fail(SAMBA_ERR_INVALID_ARG, "%s: ldo=%d must be >= N=%d", fn, ldo, N);
    const bool add = epilogue == SAMBA_GEMM_ADD_F32;
    const size_t esz = add ? 4 : 2;
    const int Nw = epilogue == SAMBA_GEMM_SWIGLU ? 2 * N : N;
    // every row and tile offset is a 32-bit byte offset from a tile base
    if (static_cast<size_t>(lda) * 2 * 256 > 0x7fffffffull || static_cast<size_t>(K) * 2 * 256 > 0x7fffffffull ||
        static_cast<size_t>(Nw) > 0x7fffffffull)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: K=%d or lda=%d too large", fn, K, lda);
    if (K > 0) {
        REQUIRE_PTR(A, "A");
        REQUIRE_PTR(W, "W");
    }
    // the epilogue stores single elements: out and residual need only element alignment
    if (out == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if ((reinterpret_cast<uintptr_t>(out) & (esz - 1)) != 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: out is not %zu-byte aligned", fn, esz);
    if (add) {
        if (residual == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: residual is NULL", fn);
        if ((reinterpret_cast<uintptr_t>(residual) & 3u) != 0)
            return fail(SAMBA_ERR_INVALID_ARG, "%s: residual is not 4-byte aligned", fn);
        if (ldr < N) return fail(SAMBA_ERR_INVALID_ARG, "%s: ldr=%d must be >= N=%d", fn, ldr, N);
    }
    const size_t a_bytes = (static_cast<size_t>(M - 1) * lda + K) * 2;
    const size_t w_bytes = static_cast<size_t>(Nw) * K * 2;
    const size_t o_bytes = (static_cast<size_t>(M - 1) * ldo + N) * esz;
    if (overlaps(out, o_bytes, A, K > 0 ? a_bytes : 0) || overlaps(out, o_bytes, W, w_bytes))
        return fail(SAMBA_ERR_INVALID_ARG, "%s: out overlaps an input", fn);
    if (add && static_cast<const void *>(residual) != out &&
        overlaps(out, o_bytes, residual, (static_cast<size_t>(M - 1) * ldr + N) * 4))
        return fail(SAMBA_ERR_INVALID_ARG, "%s: residual partially overlaps out", fn);
    if (add && static_cast<const void *>(residual) == out && ldr != ldo)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: residual is out with ldr != ldo", fn);
    const samba::gemm::Plan pl = samba::gemm::plan(M, N, K, static_cast<int>(epilogue));
    if (pl.part_bytes > 0) {
        if (workspace == nullptr || workspace_bytes < pl.part_bytes)
            return fail(SAMBA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, pl.part_bytes,
                        workspace == nullptr ? (size_t)0 : workspace_bytes);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(SAMBA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
        if (overlaps(out, o_bytes, workspace, pl.part_bytes))
            return fail(SAMBA_ERR_INVALID_ARG, "%s: out overlaps the workspace", fn);
    }
    if (static_cast<long long>(pl.tiles_m) * pl.tiles_n * pl.splits > 0x7fffffffll)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: too many tiles", fn);
    samba::gemm::GemmArgs a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.A = static_cast<const uint16_t *>(A);
    a.lda = lda;
    a.W = static_cast<const uint16_t *>(W);
    a.out = out;
    a.ldo = ldo;
    a.R = residual;
    a.ldr = ldr;
    a.part = static_cast<float *>(workspace);
    if (fz != nullptr) {
        a.nw = fz->norm_w;
        a.neps = fz->norm_eps;
        a.nout = fz->norm_out;
        a.cw = fz->conv_w;
        a.cb = fz->conv_b;
        a.c0 = fz->conv0;
        a.chead = fz->conv_head;
        a.cu = fz->conv_u;
        a.cD = fz->conv_D;
    }
    if (!samba::gemm::launch_gemm(a, static_cast<int>(epilogue), pl, static_cast<hipStream_t>(stream),
                                  fz != nullptr ? &fz->normed : nullptr, fz != nullptr ? &fz->conved : nullptr))
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: no kernel for this tile plan", fn);
    return launched(fn);
}
}  // namespace

samba_status samba_gemm(int M, int N, int K, samba_gemm_epilogue epilogue, const void *A, int lda, const void *W,
                        void *out, int ldo, const float *residual, int ldr, void *workspace, size_t workspace_bytes,
                        void *stream)
{
    return gemm_impl(M, N, K, epilogue, A, lda, W, out, ldo, residual, ldr, workspace, workspace_bytes, stream);
}

samba_status samba_rmsnorm(int rows, int d, const float *x, const float *weight, float eps, void *out, void *stream)
{
    const char *fn = "samba_rmsnorm";
    if (rows < 0 || d < 1) return fail(SAMBA_ERR_INVALID_ARG, "%s: rows=%d must be >= 0 and d=%d >= 1", fn, rows, d);
    if (!(eps >= 0.0f)) return fail(SAMBA_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
    if (rows == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(weight, "weight");
    if (out == nullptr || (reinterpret_cast<uintptr_t>(out) & 1u) != 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: out is NULL or not 2-byte aligned", fn);
    const size_t n = static_cast<size_t>(rows) * d;
    if (overlaps(out, n * 2, x, n * 4)) return fail(SAMBA_ERR_INVALID_ARG, "%s: out overlaps x", fn);
    samba::step::launch_rmsnorm(rows, d, x, weight, eps, static_cast<uint16_t *>(out), static_cast<hipStream_t>(stream));
    return launched(fn);
}

}  // extern "C"

namespace {

// Byte offsets of the decode step's intermediate activations in the caller's workspace.
// Projections that read the same input are one GEMM over concatenated weights: x and z are the
// two column halves of xz, (U W_r, B, C) the column blocks of xp, q / k / v those of qkv.
struct StepLayout {
    size_t hn, xz, u, xp, dt, y, qkv, o, m, part, swa, total;
    size_t part_bytes, swa_bytes;
};

int xproj_width(const samba_model_config &c) { return c.dt_rank + 2 * c.d_state; }
int qkv_width(const samba_model_config &c) { return (c.n_heads + 2 * c.n_kv_heads) * c.head_dim; }

StepLayout step_layout(const samba_model_config &c, int S)
{
    StepLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~static_cast<size_t>(255);
        return o;
    };
    const size_t s = static_cast<size_t>(S), hq = static_cast<size_t>(c.n_heads) * c.head_dim;
    L.hn = take(s * c.d_model * 2);
    L.xz = take(s * 2 * c.d_inner * 2);
    L.u = take(s * c.d_inner * 2);
    L.xp = take(s * xproj_width(c) * 2);
    L.dt = take(s * c.d_inner * 2);
    L.y = take(s * c.d_inner * 2);
    L.qkv = take(s * qkv_width(c) * 2);
    L.o = take(s * hq * 2);
    L.m = take(s * c.d_ff * 2);
    using samba::gemm::plan;
    const int shapes[][3] = {{2 * c.d_inner, c.d_model, 0}, {xproj_width(c), c.d_inner, 0}, {c.d_inner, c.dt_rank, 0},
                             {c.d_model, c.d_inner, 1},     {qkv_width(c), c.d_model, 0},   {c.d_model, static_cast<int>(hq), 1},
                             {c.d_ff, c.d_model, 2},        {c.d_model, c.d_ff, 1}};
    L.part_bytes = 0;
    for (const auto &sh : shapes) L.part_bytes = std::max(L.part_bytes, plan(S, sh[0], sh[1], sh[2]).part_bytes);
    L.part = take(L.part_bytes);
    L.swa_bytes = samba::swa_decode_workspace_bytes(S, c.n_heads, c.head_dim);
    L.swa = take(L.swa_bytes);
    L.total = off;
    return L;
}

samba_status check_model_config(const char *fn, const samba_model_config *c)
{
    if (c == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: config is NULL", fn);
    if (c->d_model < 8 || c->d_inner < 8 || c->dt_rank < 8 || c->d_ff < 8 || c->d_model % 8 || c->d_inner % 8 ||
        c->dt_rank % 8 || c->d_ff % 8)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: d_model=%d d_inner=%d dt_rank=%d d_ff=%d must be positive multiples of 8",
                    fn, c->d_model, c->d_inner, c->dt_rank, c->d_ff);
    if (c->d_state != samba::kMaxState)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: d_state=%d (the decode step is built for %d)", fn, c->d_state,
                    samba::kMaxState);
    if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads != 0 || c->window < 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: heads %d / %d or window %d invalid", fn, c->n_heads, c->n_kv_heads,
                    c->window);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: head_dim=%d (64 and 128 are built)", fn, c->head_dim);
    if (c->n_heads / c->n_kv_heads > samba::swadec::kMaxGroup || c->window >= 65535 * 64)
        return fail(SAMBA_ERR_UNSUPPORTED, "%s: %d query heads per KV head or window %d beyond the built limits", fn,
                    c->n_heads / c->n_kv_heads, c->window);
    if (!(c->norm_eps >= 0.0f) || !(c->rope_base > 1.0f))
        return fail(SAMBA_ERR_INVALID_ARG, "%s: norm_eps must be >= 0 and rope_base > 1", fn);
    return SAMBA_OK;
}

}  // namespace

extern "C" {

size_t samba_decode_step_workspace_bytes(const samba_model_config *cfg, int nseq)
{
    if (nseq <= 0 || check_model_config("samba_decode_step_workspace_bytes", cfg) != SAMBA_OK) return 0;
    return step_layout(*cfg, nseq).total;
}

samba_status samba_decode_step(const samba_model_config *cfg, int n_layers, const samba_layer *layers,
                               const float *final_norm_w, int nseq, float *hidden, void *out, int32_t *pos,
                               int32_t *conv_head, void *workspace, size_t workspace_bytes, void *stream)
{
    const char *fn = "samba_decode_step";
    samba_status st = check_model_config(fn, cfg);
    if (st != SAMBA_OK) return st;
    if (n_layers < 0 || nseq < 0) return fail(SAMBA_ERR_INVALID_ARG, "%s: n_layers=%d nseq=%d must be >= 0", fn, n_layers, nseq);
    if (n_layers > 0 && layers == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: layers is NULL", fn);
    if (nseq == 0) {
        g_err.clear();
        return SAMBA_OK;
    }
    if (nseq > 65535) return fail(SAMBA_ERR_UNSUPPORTED, "%s: nseq=%d exceeds 65535", fn, nseq);
    REQUIRE_PTR(hidden, "hidden");
    if (pos == nullptr) return fail(SAMBA_ERR_INVALID_ARG, "%s: pos is NULL", fn);
    if (out != nullptr) REQUIRE_PTR(final_norm_w, "final_norm_w");
    for (int l = 0; l < n_layers; ++l) {
        if (layers[l].kind < SAMBA_LAYER_MAMBA || layers[l].kind > SAMBA_LAYER_MLP)
            return fail(SAMBA_ERR_INVALID_ARG, "%s: layer %d has unknown kind %d", fn, l, layers[l].kind);
        if (layers[l].kind == SAMBA_LAYER_MAMBA && conv_head == nullptr)
            return fail(SAMBA_ERR_INVALID_ARG, "%s: conv_head is NULL but layer %d is a Mamba layer", fn, l);
    }
    if ((reinterpret_cast<uintptr_t>(conv_head) & 3u) != 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: conv_head is not 4-byte aligned", fn);
    const samba_model_config &c = *cfg;
    const StepLayout L = step_layout(c, nseq);
    if (workspace == nullptr || workspace_bytes < L.total)
        return fail(SAMBA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, L.total,
                    workspace == nullptr ? (size_t)0 : workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(SAMBA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
    char *ws = static_cast<char *>(workspace);
    uint16_t *hn = reinterpret_cast<uint16_t *>(ws + L.hn), *xz = reinterpret_cast<uint16_t *>(ws + L.xz),
             *u = reinterpret_cast<uint16_t *>(ws + L.u), *xp = reinterpret_cast<uint16_t *>(ws + L.xp),
             *dt = reinterpret_cast<uint16_t *>(ws + L.dt), *y = reinterpret_cast<uint16_t *>(ws + L.y),
             *qkv = reinterpret_cast<uint16_t *>(ws + L.qkv), *o = reinterpret_cast<uint16_t *>(ws + L.o),
             *m = reinterpret_cast<uint16_t *>(ws + L.m);
    void *part = ws + L.part, *swa = ws + L.swa;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const int S = nseq, dm = c.d_model, de = c.d_inner, dr = c.dt_rank, N = c.d_state;
    const int hq = c.n_heads * c.head_dim, hk = c.n_kv_heads * c.head_dim, wx = xproj_width(c), wq = qkv_width(c);
    int layer = -1;
    const char *what = "";
    // Runs one sub-call; a failure is reported with the layer and the step that failed.
#define STEP(name, call)                                                                               \
    do {                                                                                               \
        what = name;                                                                                   \
        const samba_status s_ = (call);                                                                \
        if (s_ != SAMBA_OK) {                                                                          \
            const std::string msg = g_err;                                                             \
            return fail(s_, "%s: layer %d (%s): %s", fn, layer, what, msg.c_str());                    \
        }                                                                                              \
    } while (0)
#define NEED(p, name)                                                                                  \
    do {                                                                                               \
        if ((p) == nullptr || !aligned16(p))                                                           \
            return fail(SAMBA_ERR_INVALID_ARG, "%s: layer %d: %s is NULL or not 16-byte aligned", fn, layer, name); \
    } while (0)
    auto gemm = [&](int Nn, int K, samba_gemm_epilogue e, const void *A, int lda, const void *W, void *dst, int ld) {
        return samba_gemm(S, Nn, K, e, A, lda, W, dst, ld, e == SAMBA_GEMM_ADD_F32 ? hidden : nullptr, ld, part,
                          L.part_bytes, stream);
    };
    // The add that ends a layer also writes the RMSNorm of the new hidden rows that the next
    // layer (or the final norm) reads, when its K range is split (the reduce then does both);
    // normed_next records whether it did.
    // SAMBA_DECODE_NOFUSE set: every reduce does only its own work (the same results, for tests)
    const bool fuse = getenv("SAMBA_DECODE_NOFUSE") == nullptr;
    bool normed_next = false;
    auto gemm_add = [&](int K, const void *A, int lda, const void *W) {
        GemmFuse fz;
        fz.norm_eps = c.norm_eps;
        if (layer + 1 < n_layers) {
            fz.norm_w = layers[layer + 1].norm_w;
            fz.norm_out = hn;
        } else if (out != nullptr) {
            fz.norm_w = final_norm_w;
            fz.norm_out = static_cast<uint16_t *>(out);
        }
        const samba_status st = gemm_impl(S, dm, K, SAMBA_GEMM_ADD_F32, A, lda, W, hidden, dm, hidden, dm, part,
                                          L.part_bytes, stream, fuse ? &fz : nullptr);
        normed_next = fz.normed;
        return st;
    };
    for (layer = 0; layer < n_layers; ++layer) {
        const samba_layer &ly = layers[layer];
        if (!normed_next) STEP("rmsnorm", samba_rmsnorm(S, dm, hidden, ly.norm_w, c.norm_eps, hn, stream));
        normed_next = false;
        if (ly.kind == SAMBA_LAYER_MAMBA) {
            NEED(ly.ssm.A, "ssm.A");
            NEED(ly.ssm.conv_w, "ssm.conv_w");
            NEED(ly.h, "h");
            NEED(ly.conv_state, "conv_state");
            // [x | z] = X [W_in ; W_g], and (by the split-K reduce, when it can) u = SiLU(conv(x))
            // for the Delta / B / C projections; the conv state is not advanced
            GemmFuse fz;
            fz.conv_w = ly.ssm.conv_w;
            fz.conv_b = ly.ssm.conv_b;
            fz.conv0 = static_cast<const uint16_t *>(ly.conv_state);
            fz.conv_head = conv_head;
            fz.conv_u = u;
            fz.conv_D = de;
            STEP("[x | z] = X [W_in; W_g]", gemm_impl(S, 2 * de, dm, SAMBA_GEMM_STORE, hn, dm, ly.w_in_gate, xz, 2 * de,
                                                       nullptr, 2 * de, part, L.part_bytes, stream, fuse ? &fz : nullptr));
            samba::ConvArgs ca{};
            ca.nseq = S;
            ca.seqlen = 1;
            ca.D = de;
            ca.x = xz;
            ca.ldx = 2 * de;
            ca.conv_w = ly.ssm.conv_w;
            ca.conv_b = ly.ssm.conv_b;
            ca.conv0 = ly.conv_state;
            ca.conv_head = conv_head;
            ca.u = u;
            if (!fz.conved) {
                samba::launch_conv_silu(ca, SAMBA_BF16, hs);
                STEP("u = SiLU(conv(x))", launched(fn));
            }
            // [U W_r | B | C] = U [W_r; W_b; W_c], then Delta's input (U W_r) W_q
            STEP("U [W_r; W_b; W_c]", gemm(wx, de, SAMBA_GEMM_STORE, u, de, ly.w_xproj, xp, wx));
            STEP("dt = (U W_r) W_q", gemm(de, dr, SAMBA_GEMM_STORE, xp, wx, ly.w_dt_up, dt, de));
            samba::ScanArgs sa = make_args(S, 1, nullptr, de, N, xz, dt, xp + dr, xp + dr + N, xz + de, &ly.ssm,
                                           ly.h, ly.conv_state, y, ly.h, ly.conv_state);
            sa.ldx = 2 * de;
            sa.ldbc = wx;
            sa.head_in = conv_head;  // advanced once for all layers at the end of the step
            sa.head_out = nullptr;
            samba::launch_decode16(sa, SAMBA_BF16, hs);
            STEP("scan decode", launched(fn));
            STEP("hidden += Y W_out", gemm_add(de, y, de, ly.w_out));
        } else if (ly.kind == SAMBA_LAYER_SWA) {
            NEED(ly.k_cache, "k_cache");
            NEED(ly.v_cache, "v_cache");
            STEP("[q | k | v] = X [W_q; W_k; W_v]", gemm(wq, dm, SAMBA_GEMM_STORE, hn, dm, ly.w_qkv, qkv, wq));
            samba::SwaDecArgs aa = swa_dec_args(S, c.n_heads, c.n_kv_heads, c.head_dim, c.window, c.rope_base, qkv,
                                                qkv + hq, qkv + hq + hk, pos, ly.k_cache, ly.v_cache, o, swa);
            aa.ldq = wq;
            aa.ldkv = wq;
            samba::launch_swa_decode(aa, hs);
            STEP("attention decode", launched(fn));
            STEP("hidden += O W_o", gemm_add(hq, o, hq, ly.w_o));
        } else {
            STEP("SwiGLU", gemm(c.d_ff, dm, SAMBA_GEMM_SWIGLU, hn, dm, ly.w12, m, c.d_ff));
            STEP("hidden += M W_3", gemm_add(c.d_ff, m, c.d_ff, ly.w3));
        }
    }
#undef NEED
    layer = n_layers;
    if (out != nullptr && !normed_next)
        STEP("final rmsnorm", samba_rmsnorm(S, dm, hidden, final_norm_w, c.norm_eps, out, stream));
#undef STEP
    samba::step::launch_advance(S, pos, conv_head, hs);
    return launched(fn);
}

}  // extern "C"
