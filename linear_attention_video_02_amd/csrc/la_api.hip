// C ABI of the ReLU linear-attention library: argument checks, launch
// configuration and dispatch.  Declarations and the full contract are in
// include/la.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "la.h"
#include "la_apply.h"
#include "la_causal.h"
#include "la_common.h"
#include "la_state.h"
#include "la_tconv.h"

// A plain copy, one 16-byte piece per lane and one workgroup per 4 KB (the
// fastest of the simple forms measured: grid-stride loops with 1 or 4 pieces
// per iteration, with or without streaming stores, were 3-17% slower): the
// reference for the practical HBM ceiling of a read + write stream
// (la_stream_copy).
__global__ __launch_bounds__(256) void la_copy_kernel(const u32x4* src, u32x4* dst, size_t n16) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) dst[i] = src[i];
}

namespace {

constexpr int kMaxPartials = 64;         // state workgroups per (batch, head), upper bound
constexpr size_t kLdsLimit = 160 * 1024; // gfx950 LDS per workgroup
constexpr size_t kFusedCombineBytes = 256 * 1024;  // per-head partials summed in the state launch

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int env_flag(const char* name, int dflt) {
    const char* s = getenv(name);
    return (s && *s) ? atoi(s) : dflt;
}

int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    const int v = atoi(s);
    return v > 0 ? v : dflt;  // only positive overrides (workgroup counts)
}

struct WsLayout {
    size_t ticket, partial, state, total;
};

WsLayout ws_layout(int BH, int d) {
    WsLayout L;
    L.ticket = 0;
    L.partial = align_up((size_t)BH * 4, 256);
    L.state = L.partial + align_up((size_t)BH * kMaxPartials * (d * d + d) * 4, 256);
    L.total = L.state + align_up((size_t)BH * (d * d + d) * 4, 256);
    return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Checks shared by every entry point.  N is the whole sequence length.
int check_common(int B, int H, int N, int d, int gt, int gh, int gw, float eps, int dtype) {
    if (dtype != LA_FP32 && dtype != LA_BF16) return LA_E_UNSUPPORTED;
    if (d != 32 && d != 64 && d != 112 && d != 128) return LA_E_UNSUPPORTED;
    if (B < 1 || H < 1 || N < 0) return LA_E_SHAPE;
    if (!(eps >= 0.0f) || eps != eps) return LA_E_SHAPE;
    const long long BH = (long long)B * H;
    if (BH > 65535) return LA_E_SHAPE;                       // grid.y limit
    if (BH * (long long)N * d >= (1ll << 40)) return LA_E_SHAPE;
    if (N >= (1 << 30)) return LA_E_SHAPE;
    const bool none = gt == 0 && gh == 0 && gw == 0;
    if (!none) {
        if (gt < 1 || gh < 1 || gw < 1) return LA_E_SHAPE;
        if ((long long)gt * gh * gw < N) return LA_E_SHAPE;
        if ((long long)gt * gh * gw >= (1ll << 31)) return LA_E_SHAPE;
    }
    return LA_OK;
}

LaGeom make_geom(int B, int H, int ntok, int n_offset, int d, int gt, int gh, int gw) {
    LaGeom g;
    memset(&g, 0, sizeof(g));
    g.BH = B * H;
    g.ntok = ntok;
    g.n_offset = n_offset;
    g.rope = !(gt == 0 && gh == 0 && gw == 0);
    if (g.rope) {
        const int P = d / 2;
        g.ph = g.pw = P / 3;
        g.pt = P - 2 * (P / 3);
        g.gh = gh;
        g.gw = gw;
        g.div_hw = make_fastdiv((uint32_t)gh * (uint32_t)gw);
        g.div_w = make_fastdiv((uint32_t)gw);
        g.div_pt = make_fastdiv((uint32_t)g.pt);
        g.div_ph = make_fastdiv((uint32_t)g.ph);
        g.div_pw = make_fastdiv((uint32_t)g.pw);
    } else {
        g.gh = g.gw = 1;
        g.div_hw = make_fastdiv(1);
        g.div_w = make_fastdiv(1);
        g.div_pt = g.div_ph = g.div_pw = make_fastdiv(1);
    }
    return g;
}

// 8-byte LDS slots of the per-workgroup RoPE table for a chunk of `chunk`
// tokens, plus the d/2 frequencies stored after it while it is built.
size_t table_entries(const LaGeom& g, int chunk) {
    if (!g.rope) return 0;
    const long long hw = (long long)g.gh * g.gw;
    const long long nt = (chunk + hw - 1) / hw + 1;   // frames one chunk can touch
    return (size_t)(nt * g.pt + (long long)g.gh * g.ph + (long long)g.gw * g.pw + g.pt + g.ph + g.pw);
}

int state_fixed_lds(int d, int dtype) {
    if (dtype == LA_BF16) {
        switch (d) {
            case 32: return StateBf16Cfg<32>::SMEM_FIXED;
            case 64: return StateBf16Cfg<64>::SMEM_FIXED;
            case 112: return StateBf16Cfg<112>::SMEM_FIXED;
            default: return StateBf16Cfg<128>::SMEM_FIXED;
        }
    }
    switch (d) {
        case 32: return StateF32Cfg<32>::SMEM_FIXED;
        case 64: return StateF32Cfg<64>::SMEM_FIXED;
        case 112: return StateF32Cfg<112>::SMEM_FIXED;
        default: return StateF32Cfg<128>::SMEM_FIXED;
    }
}

int apply_fixed_lds(int d, int dtype) {
    if (dtype == LA_BF16) {
        switch (d) {
            case 32: return ApplyBf16Cfg<32>::FIXED;
            case 64: return ApplyBf16Cfg<64>::FIXED;
            case 112: return ApplyBf16Cfg<112>::FIXED;
            default: return ApplyBf16Cfg<128>::FIXED;
        }
    }
    switch (d) {
        case 32: return ApplyF32Cfg<32>::SMEM_FIXED;
        case 64: return ApplyF32Cfg<64>::SMEM_FIXED;
        case 112: return ApplyF32Cfg<112>::SMEM_FIXED;
        default: return ApplyF32Cfg<128>::SMEM_FIXED;
    }
}

struct Plan {
    int P, chunk;
    size_t lds;
};

// State pass: about LA_STATE_WGS workgroups in all (default: one 512-thread
// workgroup per CU for bf16),
// chunks a multiple of the 64-token tile, at most kMaxPartials per head.
int plan_state(const LaGeom& g, int d, int dtype, Plan* out, int force_chunk = 0, int fixed_lds = 0) {
    if (force_chunk > 0) {  // chunking imposed by the caller (token-causal pass)
        const int P = g.ntok > 0 ? (g.ntok + force_chunk - 1) / force_chunk : 1;
        const size_t lds = (size_t)(fixed_lds > 0 ? fixed_lds : state_fixed_lds(d, dtype)) +
                           table_entries(g, force_chunk) * 8;
        if (P > kMaxPartials || lds > kLdsLimit) return LA_E_UNSUPPORTED;
        out->P = P;
        out->chunk = force_chunk;
        out->lds = lds;
        return LA_OK;
    }
    const int target = env_int("LA_STATE_WGS", dtype == LA_BF16 ? 256 : 1024);
    // chunks are whole tiles (the kernel's ring then runs on to a whole round
    // with zero tiles: a little compute, no memory traffic)
    const int tile = dtype == LA_BF16 ? (d == 32   ? StateBf16Cfg<32>::TT
                                         : d == 64  ? StateBf16Cfg<64>::TT
                                         : d == 112 ? StateBf16Cfg<112>::TT
                                                    : StateBf16Cfg<128>::TT)
                                      : 64;
    const int ntok = g.ntok;
    // at most `target` workgroups: one more than the CUs would run a second
    // wave of workgroups after the first and double the pass
    int P = target / g.BH;
    P = P < 1 ? 1 : (P > kMaxPartials ? kMaxPartials : P);
    const int max_p = ntok > 0 ? (ntok + tile - 1) / tile : 1;
    if (P > max_p) P = max_p;
    for (;;) {
        int chunk = ntok > 0 ? (ntok + P - 1) / P : tile;
        chunk = (int)align_up((size_t)chunk, tile);
        const int Peff = ntok > 0 ? (ntok + chunk - 1) / chunk : 1;
        const size_t lds = (size_t)state_fixed_lds(d, dtype) + table_entries(g, chunk) * 8;
        if (lds <= kLdsLimit) {
            out->P = Peff;
            out->chunk = chunk;
            out->lds = lds;
            return LA_OK;
        }
        if (P >= kMaxPartials || P >= max_p) return LA_E_UNSUPPORTED;   // grid plane too large
        ++P;
    }
}

// Apply pass: about LA_APPLY_WGS workgroups in all (default: one 512-thread
// workgroup per CU for bf16).
int plan_apply(const LaGeom& g, int d, int dtype, Plan* out) {
    const int target = env_int("LA_APPLY_WGS", dtype == LA_BF16 ? 256 : 1024);
    const int tile = 128;
    const int ntok = g.ntok;
    int P = target / g.BH;  // at most `target` workgroups (see plan_state)
    if (P < 1) P = 1;
    const int max_p = ntok > 0 ? (ntok + tile - 1) / tile : 1;
    if (P > max_p) P = max_p;
    for (;;) {
        int chunk = ntok > 0 ? (ntok + P - 1) / P : tile;
        chunk = (int)align_up((size_t)chunk, tile);
        const int Peff = ntok > 0 ? (ntok + chunk - 1) / chunk : 1;
        const size_t lds = (size_t)apply_fixed_lds(d, dtype) + table_entries(g, chunk) * 8;
        if (lds <= kLdsLimit) {
            out->P = Peff;
            out->chunk = chunk;
            out->lds = lds;
            return LA_OK;
        }
        if (P >= max_p) return LA_E_UNSUPPORTED;
        ++P;
    }
}

template <typename Args>
using KernelFn = void (*)(Args);

// Last HIP failure seen by this thread, for la_last_hip_error().
thread_local char g_hip_msg[256];

int hip_fail(hipError_t e, const char* what) {
    snprintf(g_hip_msg, sizeof(g_hip_msg), "%s: %s (%d): %s", what, hipGetErrorName(e), (int)e,
             hipGetErrorString(e));
    return LA_E_HIP;
}

template <typename Args>
int launch_kernel(KernelFn<Args> fn, dim3 grid, size_t lds, hipStream_t st, const Args& args,
                  int threads = 256) {
    hipError_t e = hipGetLastError();  // clear a stale error so it is not reported as ours
    (void)e;
    if (lds > 64 * 1024) {
        e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
    }
    Args copy = args;
    void* params[] = {&copy};
    e = hipLaunchKernel((const void*)fn, grid, dim3(threads), params, lds, st);
    if (e != hipSuccess) return hip_fail(e, "hipLaunchKernel");
    return LA_OK;
}

KernelFn<CombineArgs> combine_kernel(int d) {
    if (d == 32) return la_state_combine_kernel<32>;
    if (d == 64) return la_state_combine_kernel<64>;
    if (d == 112) return la_state_combine_kernel<112>;
    return la_state_combine_kernel<128>;
}

KernelFn<StateArgs> state_kernel(int d, int dtype, bool rope) {
#define LA_PICK(D)                                                                              \
    if (d == D) {                                                                               \
        if (dtype == LA_BF16) return rope ? la_state_bf16_kernel<D, true> : la_state_bf16_kernel<D, false>; \
        return rope ? la_state_f32_kernel<D, true> : la_state_f32_kernel<D, false>;             \
    }
    LA_PICK(32)
    LA_PICK(64)
    LA_PICK(112)
    LA_PICK(128)
#undef LA_PICK
    return nullptr;
}

KernelFn<ApplyArgs> apply_kernel(int d, int dtype, bool rope) {
#define LA_PICK(D)                                                                              \
    if (d == D) {                                                                               \
        if (dtype == LA_BF16) return rope ? la_apply_bf16_kernel<D, true> : la_apply_bf16_kernel<D, false>; \
        return rope ? la_apply_f32_kernel<D, true> : la_apply_f32_kernel<D, false>;             \
    }
    LA_PICK(32)
    LA_PICK(64)
    LA_PICK(112)
    LA_PICK(128)
#undef LA_PICK
    return nullptr;
}

// Enqueue the state pass over `ntok` tokens starting at global index n_offset.
int run_state(const void* K, const void* V, float* S_out, float* z_out, float* S_out2, float* z_out2,
              const float* S_carry, const float* z_carry, void* ws, int B, int H, int ntok, int n_offset,
              int d, int gt, int gh, int gw, int dtype, hipStream_t st) {
    const LaGeom g = make_geom(B, H, ntok, n_offset, d, gt, gh, gw);
    Plan pl;
    int rc = plan_state(g, d, dtype, &pl);
    if (rc != LA_OK) return rc;
    const WsLayout L = ws_layout(g.BH, d);
    CombineArgs c;
    c.partial = (float*)((char*)ws + L.partial);
    c.S_out = S_out;
    c.z_out = z_out;
    c.S_out2 = S_out2;
    c.z_out2 = z_out2;
    c.S_carry = S_carry;
    c.z_carry = z_carry;
    c.P = pl.P;
    c.BH = g.BH;
    // Stage 2 inside the state launch saves a launch but leaves each head's sum
    // to one workgroup.  That pays while a head's partials are small (P = 4 at
    // d = 64: 66 KB); with many large partials (P = 12 at d = 112: 607 KB per
    // head) the separate combine launch, spread over many workgroups, is faster.
    // LA_STATE_FUSED = 0 / 1 forces one of the two.
    const size_t head_partials = (size_t)pl.P * (size_t)(d * d + d) * 4;
    const int force = env_flag("LA_STATE_FUSED", -1);
    const bool fused = dtype == LA_BF16 && (force >= 0 ? force != 0 : head_partials <= kFusedCombineBytes);
    StateArgs a;
    a.K = K;
    a.V = V;
    a.partial = (float*)((char*)ws + L.partial);
    a.chunk = pl.chunk;
    a.P = pl.P;
    a.g = g;
    a.ticket = fused ? (unsigned*)((char*)ws + L.ticket) : nullptr;
    a.cmb = c;
    const int threads = dtype != LA_BF16 ? 256
                        : d == 32        ? StateBf16Cfg<32>::THREADS
                        : d == 64        ? StateBf16Cfg<64>::THREADS
                        : d == 112       ? StateBf16Cfg<112>::THREADS
                                         : StateBf16Cfg<128>::THREADS;
    rc = launch_kernel<StateArgs>(state_kernel(d, dtype, g.rope), dim3(pl.P * g.BH), pl.lds, st, a, threads);
    if (rc != LA_OK || fused) return rc;
    const int e4 = (d * d + d) / 4;
    return launch_kernel<CombineArgs>(combine_kernel(d), dim3((e4 + 255) / 256, g.BH), 0, st, c);
}

int run_apply(const void* Q, void* O, const float* S, const float* z, int B, int H, int ntok, int n_offset,
              int d, int gt, int gh, int gw, float eps, int dtype, hipStream_t st) {
    if (ntok == 0) return LA_OK;
    const LaGeom g = make_geom(B, H, ntok, n_offset, d, gt, gh, gw);
    Plan pl;
    int rc = plan_apply(g, d, dtype, &pl);
    if (rc != LA_OK) return rc;
    ApplyArgs a;
    a.Q = Q;
    a.O = O;
    a.S = S;
    a.z = z;
    a.eps = eps;
    a.chunk = pl.chunk;
    a.P = pl.P;
    a.ilv = 0;
    a.g = g;
    // bf16: the head's P workgroups take interleaved units of the whole head
    // instead of one contiguous chunk each, so that each head's reads and
    // writes advance as one window rather than P separate streams (3-4%
    // faster at 720p-5s; same arithmetic per token, so bitwise equal outputs).
    // LA_APPLY_ILV=0 keeps contiguous chunks.
    if (dtype == LA_BF16 && pl.P > 1 && env_flag("LA_APPLY_ILV", 1) != 0 &&
        ((size_t)ntok + (size_t)pl.P * 1024) * d * 2 < (1ull << 32)) {  // units overrun the head by < P * 1024 tokens
        const size_t lds = pl.lds - table_entries(g, pl.chunk) * 8 + table_entries(g, ntok) * 8;
        if (lds <= kLdsLimit) {
            a.ilv = 1;
            pl.lds = lds;
        }
    }
    const int threads = dtype != LA_BF16 ? 256
                        : d == 32        ? ApplyBf16Cfg<32>::THREADS
                        : d == 64        ? ApplyBf16Cfg<64>::THREADS
                        : d == 112       ? ApplyBf16Cfg<112>::THREADS
                                         : ApplyBf16Cfg<128>::THREADS;
    return launch_kernel<ApplyArgs>(apply_kernel(d, dtype, g.rope), dim3(pl.P * g.BH), pl.lds, st, a, threads);
}

// Token-causal pass: about LA_CAUSAL_WGS workgroups (default two 256-thread
// workgroups per CU), chunks a multiple of 128 tokens (the state kernel's tile
// at d = 64 and two causal steps), at most kMaxPartials per head.
int plan_causal(const LaGeom& g, Plan* out) {
    constexpr int unit = 128;
    const int target = env_int("LA_CAUSAL_WGS", 512);
    const int ntok = g.ntok;
    int P = target / g.BH;  // at most `target` workgroups (see plan_state)
    P = P < 1 ? 1 : (P > kMaxPartials ? kMaxPartials : P);
    const int max_p = (ntok + unit - 1) / unit;
    if (P > max_p) P = max_p;
    for (;;) {
        const int chunk = (int)align_up((size_t)((ntok + P - 1) / P), unit);
        const int Peff = (ntok + chunk - 1) / chunk;
        const size_t lds = (size_t)CausalBf16Cfg<64>::SMEM_FIXED + table_entries(g, chunk) * 8;
        Plan st;
        if (Peff <= kMaxPartials && lds <= kLdsLimit && plan_state(g, 64, LA_BF16, &st, chunk) == LA_OK) {
            out->P = Peff;
            out->chunk = chunk;
            out->lds = lds;
            return LA_OK;
        }
        if (P >= kMaxPartials || P >= max_p) return LA_E_UNSUPPORTED;   // grid plane too large
        ++P;
    }
}

int run_token_causal(const void* Q, const void* K, const void* V, void* O, float* S_carry, float* z_carry,
                     void* ws, int B, int H, int ntok, int n_offset, int d, int gt, int gh, int gw, float eps,
                     hipStream_t st) {
    const LaGeom g = make_geom(B, H, ntok, n_offset, d, gt, gh, gw);
    Plan pc, ps;
    int rc = plan_causal(g, &pc);
    if (rc != LA_OK) return rc;
    // Partial states in 512-thread workgroups, two per CU: the P chunks per
    // head (512 workgroups at 720p-5s) then run in one round instead of two
    // rounds of 1024-thread workgroups (235 -> 229 us per call at 720p-5s).
    // LA_TC_STATE_THREADS=1024 selects the larger workgroups.
    const bool half = env_int("LA_TC_STATE_THREADS", 512) == 512;
    rc = plan_state(g, d, LA_BF16, &ps, pc.chunk, half ? StateBf16Cfg<64, 512>::SMEM_FIXED : 0);
    if (rc != LA_OK) return rc;
    const WsLayout L = ws_layout(g.BH, d);
    float* partial = (float*)((char*)ws + L.partial);
    // 1. one partial state per chunk
    StateArgs sa;
    sa.K = K;
    sa.V = V;
    sa.partial = partial;
    sa.chunk = ps.chunk;
    sa.P = ps.P;
    sa.g = g;
    sa.ticket = nullptr;  // partials only: the prefix kernel reads them
    KernelFn<StateArgs> sk = state_kernel(d, LA_BF16, g.rope);
    if (half) sk = g.rope ? la_state_bf16_kernel<64, true, 512> : la_state_bf16_kernel<64, false, 512>;
    rc = launch_kernel<StateArgs>(sk, dim3(ps.P * g.BH), ps.lds, st, sa,
                                  half ? 512 : StateBf16Cfg<64>::THREADS);
    if (rc != LA_OK) return rc;
    // 2. exclusive prefixes in place (+ carry), total -> carry
    PrefixArgs pa;
    pa.partial = partial;
    pa.S_carry = S_carry;
    pa.z_carry = z_carry;
    pa.S_out = S_carry;
    pa.z_out = z_carry;
    pa.P = ps.P;
    rc = launch_kernel<PrefixArgs>(la_prefix_kernel<64>, dim3((d * d + d + 255) / 256, g.BH), 0, st, pa);
    if (rc != LA_OK) return rc;
    // 3. causal scan of every chunk from its prefix
    CausalArgs ca;
    ca.Q = Q;
    ca.K = K;
    ca.V = V;
    ca.O = O;
    ca.pre = partial;
    ca.eps = eps;
    ca.chunk = pc.chunk;
    ca.P = pc.P;
    ca.g = g;
    auto fn = g.rope ? la_causal_bf16_kernel<64, true> : la_causal_bf16_kernel<64, false>;
    return launch_kernel<CausalArgs>(fn, dim3(pc.P * g.BH), pc.lds, st, ca, CausalBf16Cfg<64>::THREADS);
}

size_t elem_bytes(int dtype) { return dtype == LA_BF16 ? 2 : 4; }

// Plans depend only on sizes, so a plan failure is reported before any launch.
int precheck_plans(int B, int H, int ntok, int n_offset, int d, int gt, int gh, int gw, int dtype,
                   bool state, bool apply) {
    const LaGeom g = make_geom(B, H, ntok, n_offset, d, gt, gh, gw);
    Plan pl;
    if (state) {
        int rc = plan_state(g, d, dtype, &pl);
        if (rc != LA_OK) return rc;
    }
    if (apply && ntok > 0) {
        int rc = plan_apply(g, d, dtype, &pl);
        if (rc != LA_OK) return rc;
    }
    return LA_OK;
}

}  // namespace

extern "C" {

size_t la_workspace_bytes(int B, int H, int N, int d) {
    if (check_common(B, H, N, d, 0, 0, 0, 0.0f, LA_BF16) != LA_OK) return 0;
    return ws_layout(B * H, d).total;
}

int la_state_reduce(const void* Q, const void* K, const void* V, void* O, float* S, float* z, void* ws,
                    size_t ws_bytes, int B, int H, int N, int d, int gt, int gh, int gw, int block_tokens,
                    float eps, int dtype, void* stream) {
    (void)Q;
    (void)O;
    (void)block_tokens;
    int rc = check_common(B, H, N, d, gt, gh, gw, eps, dtype);
    if (rc != LA_OK) return rc;
    if (!S || !z || !ws || (N > 0 && (!K || !V))) return LA_E_NULLPTR;
    if (!aligned16(K) || !aligned16(V) || !aligned16(S) || !aligned16(z) || !aligned16(ws)) return LA_E_ALIGN;
    if (ws_bytes < ws_layout(B * H, d).total) return LA_E_WORKSPACE;
    const size_t nS = (size_t)B * H * d * d * 4, nz = (size_t)B * H * d * 4;
    const size_t nkv = (size_t)B * H * N * d * elem_bytes(dtype);
    if (overlaps(S, nS, K, nkv) || overlaps(S, nS, V, nkv) || overlaps(z, nz, K, nkv) ||
        overlaps(z, nz, V, nkv) || overlaps(S, nS, z, nz))
        return LA_E_ALIAS;
    rc = precheck_plans(B, H, N, 0, d, gt, gh, gw, dtype, true, false);
    if (rc != LA_OK) return rc;
    return run_state(K, V, S, z, nullptr, nullptr, nullptr, nullptr, ws, B, H, N, 0, d, gt, gh, gw, dtype,
                     (hipStream_t)stream);
}

int la_apply(const void* Q, const void* K, const void* V, void* O, const float* S, const float* z, void* ws,
             size_t ws_bytes, int B, int H, int N, int d, int gt, int gh, int gw, int block_tokens, float eps,
             int dtype, void* stream) {
    (void)K;
    (void)V;
    (void)ws;
    (void)ws_bytes;
    (void)block_tokens;
    int rc = check_common(B, H, N, d, gt, gh, gw, eps, dtype);
    if (rc != LA_OK) return rc;
    if (N == 0) return LA_OK;  // nothing to write
    if (!Q || !O || !S || !z) return LA_E_NULLPTR;
    if (!aligned16(Q) || !aligned16(O) || !aligned16(S) || !aligned16(z)) return LA_E_ALIGN;
    const size_t nqo = (size_t)B * H * N * d * elem_bytes(dtype);
    if (overlaps(O, nqo, Q, nqo) || overlaps(O, nqo, S, (size_t)B * H * d * d * 4) ||
        overlaps(O, nqo, z, (size_t)B * H * d * 4))
        return LA_E_ALIAS;
    rc = precheck_plans(B, H, N, 0, d, gt, gh, gw, dtype, false, true);
    if (rc != LA_OK) return rc;
    return run_apply(Q, O, S, z, B, H, N, 0, d, gt, gh, gw, eps, dtype, (hipStream_t)stream);
}

int la_block_causal_step(const void* Q, const void* K, const void* V, void* O, float* S_carry, float* z_carry,
                         void* ws, size_t ws_bytes, int B, int H, int N, int d, int gt, int gh, int gw,
                         int block_tokens, float eps, int dtype, int block_idx, int commit, void* stream) {
    int rc = check_common(B, H, N, d, gt, gh, gw, eps, dtype);
    if (rc != LA_OK) return rc;
    if (block_tokens < 1 || block_idx < 0 || (commit != 0 && commit != 1)) return LA_E_SHAPE;
    const long long start = (long long)block_idx * block_tokens;
    if (start >= N) return LA_E_SHAPE;
    const int Lb = (int)((N - start) < block_tokens ? (N - start) : block_tokens);
    if (!Q || !K || !V || !O || !S_carry || !z_carry || !ws) return LA_E_NULLPTR;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(S_carry) ||
        !aligned16(z_carry) || !aligned16(ws))
        return LA_E_ALIGN;
    const WsLayout L = ws_layout(B * H, d);
    if (ws_bytes < L.total) return LA_E_WORKSPACE;
    const size_t nb = (size_t)B * H * Lb * d * elem_bytes(dtype);
    const size_t nS = (size_t)B * H * d * d * 4, nz = (size_t)B * H * d * 4;
    if (overlaps(O, nb, Q, nb) || overlaps(O, nb, K, nb) || overlaps(O, nb, V, nb) ||
        overlaps(O, nb, S_carry, nS) || overlaps(O, nb, z_carry, nz) || overlaps(S_carry, nS, z_carry, nz) ||
        overlaps(S_carry, nS, K, nb) || overlaps(S_carry, nS, V, nb) || overlaps(z_carry, nz, K, nb) ||
        overlaps(z_carry, nz, V, nb) || overlaps(ws, ws_bytes, S_carry, nS) || overlaps(ws, ws_bytes, z_carry, nz))
        return LA_E_ALIAS;
    rc = precheck_plans(B, H, Lb, (int)start, d, gt, gh, gw, dtype, true, true);
    if (rc != LA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    float* Sb = (float*)((char*)ws + L.state);
    float* zb = Sb + (size_t)B * H * d * d;
    rc = run_state(K, V, Sb, zb, commit ? S_carry : nullptr, commit ? z_carry : nullptr, S_carry, z_carry, ws, B,
                   H, Lb, (int)start, d, gt, gh, gw, dtype, st);
    if (rc != LA_OK) return rc;
    return run_apply(Q, O, Sb, zb, B, H, Lb, (int)start, d, gt, gh, gw, eps, dtype, st);
}

int la_token_causal(const void* Q, const void* K, const void* V, void* O, float* S_carry, float* z_carry,
                    void* ws, size_t ws_bytes, int B, int H, int N, int d, int gt, int gh, int gw, int n_offset,
                    float eps, int dtype, void* stream) {
    if (n_offset < 0 || N < 0 || (long long)n_offset + N >= (1ll << 30)) return LA_E_SHAPE;
    int rc = check_common(B, H, n_offset + N, d, gt, gh, gw, eps, dtype);
    if (rc != LA_OK) return rc;
    if (dtype != LA_BF16 || d != 64) return LA_E_UNSUPPORTED;
    if ((S_carry == nullptr) != (z_carry == nullptr)) return LA_E_NULLPTR;
    if (!ws || (N > 0 && (!Q || !K || !V || !O))) return LA_E_NULLPTR;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(ws) ||
        !aligned16(S_carry) || !aligned16(z_carry))
        return LA_E_ALIGN;
    const WsLayout L = ws_layout(B * H, d);
    if (ws_bytes < L.total) return LA_E_WORKSPACE;
    if (N == 0) return LA_OK;  // no token: the carry stays as it is
    const size_t nb = (size_t)B * H * N * d * elem_bytes(dtype);
    const size_t nS = S_carry ? (size_t)B * H * d * d * 4 : 0, nz = z_carry ? (size_t)B * H * d * 4 : 0;
    if (overlaps(O, nb, Q, nb) || overlaps(O, nb, K, nb) || overlaps(O, nb, V, nb) ||
        overlaps(O, nb, S_carry, nS) || overlaps(O, nb, z_carry, nz) || overlaps(S_carry, nS, z_carry, nz) ||
        overlaps(S_carry, nS, K, nb) || overlaps(S_carry, nS, V, nb) || overlaps(S_carry, nS, Q, nb) ||
        overlaps(z_carry, nz, K, nb) || overlaps(z_carry, nz, V, nb) || overlaps(z_carry, nz, Q, nb) ||
        overlaps(ws, ws_bytes, S_carry, nS) || overlaps(ws, ws_bytes, z_carry, nz) ||
        overlaps(ws, ws_bytes, O, nb))
        return LA_E_ALIAS;
    {
        const LaGeom g = make_geom(B, H, N, n_offset, d, gt, gh, gw);
        Plan pc;
        rc = plan_causal(g, &pc);
        if (rc != LA_OK) return rc;
    }
    return run_token_causal(Q, K, V, O, S_carry, z_carry, ws, B, H, N, n_offset, d, gt, gh, gw, eps,
                            (hipStream_t)stream);
}

int la_temporal_conv_step(const void* X, void* Y, const void* W, const float* bias, void* cache, int B, int T,
                          int P, int D, int commit, int dtype, void* stream) {
    if (dtype != LA_BF16) return LA_E_UNSUPPORTED;
    if (B < 0 || T < 0 || P < 0 || D < 1 || (commit != 0 && commit != 1)) return LA_E_SHAPE;
    if (D % 64 != 0 || D > 16384) return LA_E_UNSUPPORTED;  // W under 2 GiB
    const long long M = (long long)B * T * P;
    if (M * D * 2 >= (1ll << 31)) return LA_E_UNSUPPORTED;  // X under 2 GiB (32-bit buffer offsets)
    if (M == 0) return LA_OK;  // an empty block: no output, the cache stays
    if (!X || !Y || !W || !cache) return LA_E_NULLPTR;
    if (!aligned16(X) || !aligned16(Y) || !aligned16(W) || !aligned16(cache) || !aligned16(bias))
        return LA_E_ALIGN;
    const size_t nx = (size_t)M * D * 2, nw = (size_t)3 * D * D * 2, nc = (size_t)B * P * D * 2;
    const size_t nb = bias ? (size_t)D * 4 : 0;
    if (overlaps(Y, nx, X, nx) || overlaps(Y, nx, W, nw) || overlaps(Y, nx, cache, nc) ||
        overlaps(Y, nx, bias, nb) || overlaps(cache, nc, X, nx) || overlaps(cache, nc, W, nw) ||
        overlaps(cache, nc, bias, nb))
        return LA_E_ALIAS;
    TconvArgs a;
    a.X = (const uint16_t*)X;
    a.Y = (uint16_t*)Y;
    a.W = (const uint16_t*)W;
    a.bias = bias;
    a.cache = (const uint16_t*)cache;
    a.T = T;
    a.P = P;
    a.D = D;
    a.M = (int)M;
    a.F = T < TconvCfg::FMAX ? T : TconvCfg::FMAX;
    a.S = tconv_positions(a.F);
    a.nft = (T + a.F - 1) / a.F;
    a.npt = (P + a.S - 1) / a.S;
    if ((long long)B * a.nft * a.npt >= (1ll << 31) / 8) return LA_E_UNSUPPORTED;
    a.mtiles = B * a.nft * a.npt;
    a.ntiles = (D + TconvCfg::BN - 1) / TconvCfg::BN;
    a.gm = env_int("LA_TCONV_GM", 8);
    a.gn = env_int("LA_TCONV_GN", 7);
    if ((long long)a.mtiles * a.ntiles >= (1ll << 31)) return LA_E_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    (void)hipGetLastError();  // clear a stale error so it is not reported as ours
    hipError_t e = la_tconv_launch(a, st);
    if (e != hipSuccess) return hip_fail(e, "la_tconv_bf16_kernel launch");
    if (!commit) return LA_OK;
    TconvCacheArgs c;
    c.X = (const uint16_t*)X;
    c.cache = (uint16_t*)cache;
    c.T = T;
    c.P = P;
    c.D = D;
    c.B = B;
    e = la_tconv_cache_launch(c, st);
    if (e != hipSuccess) return hip_fail(e, "la_tconv_cache_kernel launch");
    return LA_OK;
}

int la_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes == 0) return LA_OK;
    if (!src || !dst) return LA_E_NULLPTR;
    if (!aligned16(src) || !aligned16(dst) || bytes % 16 != 0) return LA_E_ALIGN;
    if (overlaps(src, bytes, dst, bytes)) return LA_E_ALIAS;
    const size_t n16 = bytes / 16;
    const size_t blocks = (n16 + 255) / 256;
    if (blocks >= (1ull << 31)) return LA_E_UNSUPPORTED;
    const unsigned grid = (unsigned)blocks;
    (void)hipGetLastError();
    hipLaunchKernelGGL(la_copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                       (u32x4*)dst, n16);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? LA_OK : hip_fail(e, "la_copy_kernel launch");
}

const char* la_last_hip_error(void) { return g_hip_msg; }

const char* la_strerror(int status) {
    switch (status) {
        case LA_OK: return "ok";
        case LA_E_NULLPTR: return "a required pointer is NULL";
        case LA_E_SHAPE: return "invalid shape, grid or block arguments";
        case LA_E_UNSUPPORTED: return "unsupported head dim, dtype or grid size";
        case LA_E_ALIGN: return "pointer not 16-byte aligned";
        case LA_E_WORKSPACE: return "workspace too small";
        case LA_E_HIP: return "HIP runtime rejected a launch";
        case LA_E_ALIAS: return "output overlaps an input";
        default: return "unknown status";
    }
}

}  // extern "C"
