// C ABI of the ReLU linear-attention library: argument checks, launch
// configuration and dispatch.  Declarations and the full contract are in
// include/la.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "la.h"
#include "la_apply.h"
#include "la_causal.h"
#include "la_common.h"
#include "la_state.h"
#include "la_tconv.h"

// A plain copy, one 16-byte piece per lane and one workgroup per 4 KB, with
// the cache policies of the attention kernels' streams: non-temporal loads
// and streaming (sc1 nt) stores.  The fastest of the simple forms measured
// (158 MB, gfx950): 6.44 TB/s, against 5.83 with default loads and stores
// and 5.95 with non-temporal loads only; grid-stride loops with 1 or 4 pieces
// per iteration were 3-17% slower.  The reference for the practical HBM
// ceiling of a read + write stream (la_stream_copy).  Each workgroup's
// descriptors cover its own 4 KB (its tail past n16 reads zeros and is not
// stored), so any size works with 32-bit buffer offsets.
__global__ __launch_bounds__(256) void la_copy_kernel(const u32x4* src, u32x4* dst, size_t n16) {
    const size_t b0 = (size_t)blockIdx.x * 256;  // first piece of this workgroup (< n16)
    const uint32_t nb = (uint32_t)((n16 - b0 < 256 ? n16 - b0 : 256) * 16);
    const BufRsrc rs = make_rsrc(src + b0, nb);
    const BufRsrc rd = make_rsrc(dst + b0, nb);
    buf_store16_stream(buf_load16(rs, threadIdx.x * 16u), rd, threadIdx.x * 16u);
}

// Scratch of la_state_reduce_noalloc, for callers that cannot allocate: the
// same layout as a caller's workspace (counters, then partial states), in a
// fixed array of the code object.  Each GPU the library runs on holds its own
// copy until the process ends.  Host code uses the array only through the
// device address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void la_zero_kernel(u32x4* p, size_t n16) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) p[i] = u32x4{0u, 0u, 0u, 0u};
}

namespace {

constexpr int kMaxPartials = 64;         // state workgroups per (batch, head), upper bound
constexpr size_t kLdsLimit = 160 * 1024; // gfx950 LDS per workgroup
constexpr size_t kFusedCombineBytes = 256 * 1024;  // per-head partials summed in the state launch
constexpr int kOnePartTiles = 4;  // state pass: up to this many tiles a head, one workgroup per head

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Tuning knobs, for measurement only (A/B runs on one build): every knob
// starts unset, meaning the default choice, and changes only through
// la_set_tuning().  Nothing here reads the process environment.
enum Knob {
    K_STATE_WGS, K_APPLY_WGS, K_CAUSAL_WGS, K_STATE_FUSED, K_APPLY_ILV, K_APPLY_HEADS,
    K_TC_STATE_THREADS, K_TCONV_GM, K_TCONV_GN, K_APPLY_SPREAD, K_CROSS_FUSED, K_COUNT
};
struct KnobInfo {
    const char* name;
    int lo, hi;  // accepted values (a negative value resets the knob)
};
const KnobInfo kKnobs[] = {
    {"state_wgs", 1, 1 << 20},  {"apply_wgs", 1, 1 << 20},  {"causal_wgs", 1, 1 << 20},
    {"state_fused", 0, 1},      {"apply_ilv", 0, 1},        {"apply_heads", 1, 8},
    {"tc_state_threads", 512, 1024}, {"tconv_gm", 1, 64},   {"tconv_gn", 1, 64},
    {"apply_spread", 0, 1},     {"cross_fused", 0, 1},
};
static_assert(sizeof(kKnobs) / sizeof(kKnobs[0]) == K_COUNT, "one table entry per knob");
// every knob starts unset (-1), however many there are
struct KnobValues {
    int v[K_COUNT];
    KnobValues() {
        for (int& x : v) x = -1;
    }
};
KnobValues g_knob_values;
int* const g_knob = g_knob_values.v;

int knob(Knob k, int dflt) { return g_knob[k] >= 0 ? g_knob[k] : dflt; }

// Workspace: per-head stage-2 counters (64-bit, epoch-tagged, a fixed 32 KB
// region), the partial states [BH][P][d*d + d] of the state pass, then the
// block-mode sums
// S_b/z_b [BH][d*d + d].  P is the partial count of the call's plan.
struct WsLayout {
    size_t ticket, partial, state, total;
};

// The counters sit at the same place for every shape, ahead of everything
// else: a workspace shared by calls of different sizes never has one call's
// partial states land on another's counters.  The fused stage 2 (which uses
// them) is limited to kTicketHeads (batch, head) pairs.
constexpr int kTicketHeads = 4096;

WsLayout ws_layout(int BH, int d, int P) {
    WsLayout L;
    L.ticket = 0;
    L.partial = (size_t)kTicketHeads * 8;
    L.state = L.partial + align_up((size_t)BH * (size_t)P * (d * d + d) * 4, 256);
    L.total = L.state + align_up((size_t)BH * (d * d + d) * 4, 256);
    return L;
}

// Epoch of a call's counters: increases from call to call across the process
// (never 0, the value of a zero-filled workspace), so a counter a call finds
// from an earlier call -- even one that never completed -- restarts at zero.
std::atomic<unsigned> g_epoch{0};

unsigned next_epoch() {
    unsigned e = ++g_epoch;
    while (e == 0) e = ++g_epoch;
    return e;
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

// LDS of the bf16 apply: fixed part (staging tiles) and the operand buffer
// each head of a slot takes (the RoPE table comes on top), heads per slot at
// most, and the unit of work
void apply_bf16_lds(int d, int* fixed, int* perhead, int* maxph, int* unit) {
#define LA_CFG(D)                            \
    if (d == D) {                            \
        *fixed = ApplyBf16Cfg<D>::FIXED;     \
        *perhead = ApplyBf16Cfg<D>::PERHEAD; \
        *maxph = ApplyBf16Cfg<D>::MAXPH;     \
        *unit = ApplyBf16Cfg<D>::UNIT;       \
        return;                              \
    }
    LA_CFG(32)
    LA_CFG(64)
    LA_CFG(112)
    LA_CFG(128)
#undef LA_CFG
}

int apply_f32_lds(int d) {
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

// State pass: about state_wgs workgroups in all (default: one 512-thread
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
    const int target = knob(K_STATE_WGS, dtype == LA_BF16 ? 256 : 1024);
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
    // A sequence of at most kOnePartTiles tiles goes to one bf16 workgroup per
    // head, which writes S and z itself: no partials, no second stage (text
    // keys of cross-attention, short blocks).  Set state_wgs to override.
    if (dtype == LA_BF16 && knob(K_STATE_WGS, -1) < 0 && max_p <= kOnePartTiles) P = 1;
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

// Apply pass.
//  - bf16, interleaved (the default): nph heads per workgroup one after
//    another, P workgroups per head taking interleaved units of it, hs = BH /
//    nph head slots, about apply_wgs (256) workgroups in all.  The most heads
//    per workgroup (fewest heads in flight) such that nph divides BH, the
//    workgroups still fill the chip, every workgroup has at least 8 units
//    per head, and the S^T copies plus the RoPE table of the whole head fit
//    in LDS.
//  - otherwise (fp32, a table too large for LDS, or apply_ilv = 0): one
//    contiguous chunk per workgroup, P chunks per head.
struct ApplyPlan {
    int ilv, P, nph, hs, spread, chunk, grid;
    size_t lds;
};

// Heads per bf16 apply workgroup unless the apply_heads knob says otherwise.
// Measured (d = 64): the apply runs best with about 8 workgroups per slot of
// heads; one head per workgroup gets there when the target gives each head 8
// or more, else (64 heads at 720p-5s: 4 a head) two heads per workgroup do.
// Past 64 channels one (S^T of two heads fills the LDS).
int default_apply_heads(int d, int BH, int target) {
    if (d > 64) return 1;
    return target / BH >= 8 ? 1 : 2;
}

int plan_apply(const LaGeom& g, int d, int dtype, ApplyPlan* out) {
    const int target = knob(K_APPLY_WGS, dtype == LA_BF16 ? 256 : 1024);
    const int ntok = g.ntok;
    const int BH = g.BH;
    int fixed = 0, perhead = 0, maxph = 1, unit = 32;
    if (dtype == LA_BF16) apply_bf16_lds(d, &fixed, &perhead, &maxph, &unit);
    if (dtype == LA_BF16 && ntok > 0 && knob(K_APPLY_ILV, 1) != 0) {
        const int U = (ntok + unit - 1) / unit;  // units per head
        const int pmax = U / 8 > 1 ? U / 8 : 1;
        const long long want = (long long)BH * pmax < target ? (long long)BH * pmax : target;
        const size_t table = table_entries(g, ntok) * 8;
        const int forced = knob(K_APPLY_HEADS, 0);
        const int first = forced > 0 ? forced : (maxph < default_apply_heads(d, BH, target) ? maxph : default_apply_heads(d, BH, target));
        for (int nph = first; nph >= 1; --nph) {
            if (nph > maxph || BH % nph != 0) {
                if (forced > 0) break;
                continue;
            }
            const int hs = BH / nph;
            int P = target / hs;
            P = P < 1 ? 1 : (P > pmax ? pmax : P);
            // enough workgroups to fill the chip (one head per workgroup always qualifies)
            if (forced <= 0 && nph > 1 && (long long)hs * P * 10 < want * 9) continue;
            const size_t lds = (size_t)fixed + (size_t)nph * perhead + table;
            if (lds > kLdsLimit) {
                if (forced > 0) break;
                continue;
            }
            // buffer offsets of units past a head's end stay below 2^32, and
            // unit numbers fit the 20 bits of a mailbox word
            if (((size_t)ntok + (size_t)(P + 1) * unit) * d * 2 >= (1ull << 32)) break;
            if (U >= (1 << 20)) break;
            if ((long long)hs * P >= (1ll << 31)) break;
            out->ilv = 1;
            out->P = P;
            out->nph = nph;
            out->hs = hs;
            // a slot's workgroups on all 8 XCDs (workgroup i runs on XCD i % 8),
            // or on as few as possible.  Measured: at d <= 64 few XCDs per slot are
            // faster (N = 65,536, 32 heads: 99 against 109 us; 720p-5s 63.2
            // against 64.3 us), at d = 128 all eight slightly (231 against 235 us).
            out->spread = P % 8 == 0 && knob(K_APPLY_SPREAD, d > 64 ? 1 : 0) != 0;
            out->chunk = ntok;
            out->grid = hs * P;
            out->lds = lds;
            return LA_OK;
        }
    }
    const int tile = 128;
    int P = target / BH;  // at most `target` workgroups (see plan_state)
    if (P < 1) P = 1;
    const int max_p = ntok > 0 ? (ntok + tile - 1) / tile : 1;
    if (P > max_p) P = max_p;
    // A sequence of at most kOnePartTiles tiles goes to one bf16 workgroup per
    // head, which writes S and z itself: no partials, no second stage (text
    // keys of cross-attention, short blocks).  Set state_wgs to override.
    if (dtype == LA_BF16 && knob(K_STATE_WGS, -1) < 0 && max_p <= kOnePartTiles) P = 1;
    for (;;) {
        int chunk = ntok > 0 ? (ntok + P - 1) / P : tile;
        chunk = (int)align_up((size_t)chunk, tile);
        const int Peff = ntok > 0 ? (ntok + chunk - 1) / chunk : 1;
        const size_t base = dtype == LA_BF16 ? (size_t)fixed + perhead : (size_t)apply_f32_lds(d);
        const size_t lds = base + table_entries(g, chunk) * 8;
        // a chunk's byte range and unit numbers fit 32-bit offsets and 20-bit words
        const bool small = ((size_t)chunk + 2 * (size_t)tile) * d * 4 < (1ull << 32) && chunk / unit < (1 << 20);
        if (lds <= kLdsLimit && small) {
            if ((long long)Peff * BH >= (1ll << 31)) return LA_E_UNSUPPORTED;
            out->ilv = 0;
            out->P = Peff;
            out->nph = 1;
            out->hs = BH;
            out->spread = 0;
            out->chunk = chunk;
            out->grid = Peff * BH;
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

// bf16: the instance with the fewest S register slots that holds nph heads
template <int D, bool ROPE>
KernelFn<ApplyArgs> apply_bf16_kernel(int nph) {
    constexpr int M = ApplyBf16Cfg<D>::MAXPH;
    if (nph <= 1) return la_apply_bf16_kernel<D, ROPE, 1>;
    if (nph <= 2 || M <= 2) return la_apply_bf16_kernel<D, ROPE, (M < 2 ? M : 2)>;
    return la_apply_bf16_kernel<D, ROPE, M>;
}

// cross-attention in one launch (d = 64, no RoPE): the KV instance with one or two heads
KernelFn<ApplyArgs> apply_kv_kernel(int nph) {
    return nph <= 1 ? la_apply_bf16_kernel<64, false, 1, true> : la_apply_bf16_kernel<64, false, 2, true>;
}

KernelFn<ApplyArgs> apply_kernel(int d, int dtype, bool rope, int nph) {
#define LA_PICK(D)                                                                              \
    if (d == D) {                                                                               \
        if (dtype == LA_BF16) return rope ? apply_bf16_kernel<D, true>(nph) : apply_bf16_kernel<D, false>(nph); \
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
    const WsLayout L = ws_layout(g.BH, d, pl.P);
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
    // The tuning knob state_fused = 0 / 1 forces one of the two.
    const size_t head_partials = (size_t)pl.P * (size_t)(d * d + d) * 4;
    const int force = knob(K_STATE_FUSED, -1);
    const bool fused = dtype == LA_BF16 && g.BH <= kTicketHeads &&
                       (force >= 0 ? force != 0 : head_partials <= kFusedCombineBytes);
    StateArgs a;
    a.K = K;
    a.V = V;
    a.partial = (float*)((char*)ws + L.partial);
    a.chunk = pl.chunk;
    a.P = pl.P;
    a.pslots = pl.P;
    a.g = g;
    a.ticket = fused ? (unsigned long long*)((char*)ws + L.ticket) : nullptr;
    a.epoch = next_epoch();
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
    ApplyPlan pl;
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
    a.ilv = pl.ilv;
    a.nph = pl.nph;
    a.hs = pl.hs;
    a.spread = pl.spread;
    a.g = g;
    a.K = nullptr;
    a.V = nullptr;
    a.nkv = 0;
    const int threads = dtype != LA_BF16 ? 256
                        : d == 32        ? ApplyBf16Cfg<32>::THREADS
                        : d == 64        ? ApplyBf16Cfg<64>::THREADS
                        : d == 112       ? ApplyBf16Cfg<112>::THREADS
                                         : ApplyBf16Cfg<128>::THREADS;
    return launch_kernel<ApplyArgs>(apply_kernel(d, dtype, g.rope, pl.nph), dim3(pl.grid), pl.lds, st, a, threads);
}

// Linear cross-attention in one launch: the apply kernel's KV instance forms
// each head's S and z from its n_kv keys/values (bf16, d = 64, n_kv <=
// KV_MAXKV).  Returns LA_E_UNSUPPORTED, launching nothing, where the
// plan puts more than two heads on a workgroup.
int run_cross_fused(const void* Q, const void* K, const void* V, void* O, int B, int H, int nq, int nkv, float eps,
                    hipStream_t st) {
    const LaGeom g = make_geom(B, H, nq, 0, 64, 0, 0, 0);
    ApplyPlan pl;
    int rc = plan_apply(g, 64, LA_BF16, &pl);
    if (rc != LA_OK) return rc;
    if (pl.nph > 2 || nkv > KV_MAXKV) return LA_E_UNSUPPORTED;
    ApplyArgs a;
    a.Q = Q;
    a.O = O;
    a.S = nullptr;
    a.z = nullptr;
    a.K = K;
    a.V = V;
    a.nkv = nkv;
    a.eps = eps;
    a.chunk = pl.chunk;
    a.P = pl.P;
    a.ilv = pl.ilv;
    a.nph = pl.nph;
    a.hs = pl.hs;
    a.spread = pl.spread;
    a.g = g;
    return launch_kernel<ApplyArgs>(apply_kv_kernel(pl.nph), dim3(pl.grid), pl.lds, st, a,
                                    ApplyBf16Cfg<64>::THREADS);
}

// Cross-attention workspace: the state pass's over n_kv tokens, then S and z
// (used where the two-launch path runs)
size_t cross_ws_bytes(int BH, int d, int partials) {
    return align_up(ws_layout(BH, d, partials).total, 256) + align_up((size_t)BH * d * d * 4, 256) +
           align_up((size_t)BH * d * 4, 256);
}

// LDS of the token-causal scan kernel without its RoPE table
size_t causal_fixed_lds(int d, int dtype) {
#define LA_CFG(D)                                                                                  \
    if (d == D) return dtype == LA_BF16 ? (size_t)CausalBf16Cfg<D>::SMEM_FIXED : (size_t)CausalF32Cfg<D>::SMEM_FIXED;
    LA_CFG(32)
    LA_CFG(64)
    LA_CFG(112)
#undef LA_CFG
    return dtype == LA_BF16 ? (size_t)CausalBf16Cfg<128>::SMEM_FIXED : (size_t)CausalF32Cfg<128>::SMEM_FIXED;
}

// The partial-state pass of token-causal mode: at bf16 d = 64 the 512-thread
// state kernel, two per CU (see run_token_causal), unless the tuning knob
// tc_state_threads = 1024 asks for the larger workgroups.
bool tc_half_state(int d, int dtype) {
    return dtype == LA_BF16 && d == 64 && knob(K_TC_STATE_THREADS, 512) == 512;
}

// Token-causal pass: about causal_wgs workgroups (default two 256-thread
// workgroups per CU where two fit -- bf16, d <= 64 -- else one), chunks a
// multiple of 128 tokens (the state kernel's tile at d = 64 and two causal
// steps), at most kMaxPartials per head.
int plan_causal(const LaGeom& g, int d, int dtype, Plan* out) {
    constexpr int unit = 128;
    const bool two_per_cu = dtype == LA_BF16 && d <= 64;
    const int target = knob(K_CAUSAL_WGS, two_per_cu ? 512 : 256);
    const int ntok = g.ntok;
    int P = target / g.BH;  // at most `target` workgroups (see plan_state)
    P = P < 1 ? 1 : (P > kMaxPartials ? kMaxPartials : P);
    const int max_p = (ntok + unit - 1) / unit;
    if (P > max_p) P = max_p;
    const int state_lds = tc_half_state(d, dtype) ? StateBf16Cfg<64, 512>::SMEM_FIXED : 0;
    for (;;) {
        const int chunk = (int)align_up((size_t)((ntok + P - 1) / P), unit);
        const int Peff = (ntok + chunk - 1) / chunk;
        const size_t lds = causal_fixed_lds(d, dtype) + table_entries(g, chunk) * 8;
        Plan st;
        if (Peff <= kMaxPartials && lds <= kLdsLimit && plan_state(g, d, dtype, &st, chunk, state_lds) == LA_OK) {
            out->P = Peff;
            out->chunk = chunk;
            out->lds = lds;
            return LA_OK;
        }
        if (P >= kMaxPartials || P >= max_p) return LA_E_UNSUPPORTED;   // grid plane too large
        ++P;
    }
}

KernelFn<CausalArgs> causal_kernel(int d, int dtype, bool rope) {
#define LA_PICK(D)                                                                                  \
    if (d == D) {                                                                                   \
        if (dtype == LA_BF16) return rope ? la_causal_bf16_kernel<D, true> : la_causal_bf16_kernel<D, false>; \
        return rope ? la_causal_f32_kernel<D, true> : la_causal_f32_kernel<D, false>;             \
    }
    LA_PICK(32)
    LA_PICK(64)
    LA_PICK(112)
    LA_PICK(128)
#undef LA_PICK
    return nullptr;
}

KernelFn<PrefixArgs> prefix_kernel(int d) {
    if (d == 32) return la_prefix_kernel<32>;
    if (d == 64) return la_prefix_kernel<64>;
    if (d == 112) return la_prefix_kernel<112>;
    return la_prefix_kernel<128>;
}

int state_threads(int d, int dtype) {
    return dtype != LA_BF16 ? 256
           : d == 32        ? StateBf16Cfg<32>::THREADS
           : d == 64        ? StateBf16Cfg<64>::THREADS
           : d == 112       ? StateBf16Cfg<112>::THREADS
                            : StateBf16Cfg<128>::THREADS;
}

// Token-causal mode (Eq. 3 token by token): partial states of the chunks,
// their exclusive prefixes in place, then the causal scan of every chunk.
int run_token_causal(const void* Q, const void* K, const void* V, void* O, float* S_carry, float* z_carry,
                     void* ws, int B, int H, int ntok, int n_offset, int d, int gt, int gh, int gw, float eps,
                     int dtype, hipStream_t st) {
    const LaGeom g = make_geom(B, H, ntok, n_offset, d, gt, gh, gw);
    Plan pc, ps;
    int rc = plan_causal(g, d, dtype, &pc);
    if (rc != LA_OK) return rc;
    // bf16 d = 64: partial states in 512-thread workgroups, two per CU: the P
    // chunks per head (512 workgroups at 720p-5s) then run in one round
    // instead of two rounds of 1024-thread workgroups (235 -> 229 us per call
    // at 720p-5s).
    const bool half = tc_half_state(d, dtype);
    rc = plan_state(g, d, dtype, &ps, pc.chunk, half ? StateBf16Cfg<64, 512>::SMEM_FIXED : 0);
    if (rc != LA_OK) return rc;
    const WsLayout L = ws_layout(g.BH, d, ps.P);
    float* partial = (float*)((char*)ws + L.partial);
    // 1. one partial state per chunk.  Without a carry to return, no prefix
    // needs the last chunk's sum (the scan of that chunk starts from the sum
    // of the ones before it), so its partial is not computed: the prefix
    // kernel then writes the exclusive prefixes as before, and only the
    // total, which is not stored, would have used that slot.
    StateArgs sa;
    sa.K = K;
    sa.V = V;
    sa.partial = partial;
    sa.chunk = ps.chunk;
    sa.P = S_carry ? ps.P : ps.P - 1;
    sa.pslots = ps.P;
    sa.g = g;
    sa.ticket = nullptr;  // partials only: the prefix kernel reads them
    sa.epoch = 0;
    KernelFn<StateArgs> sk = state_kernel(d, dtype, g.rope);
    if (half) sk = g.rope ? la_state_bf16_kernel<64, true, 512> : la_state_bf16_kernel<64, false, 512>;
    if (sa.P > 0) {
        rc = launch_kernel<StateArgs>(sk, dim3(sa.P * g.BH), ps.lds, st, sa, half ? 512 : state_threads(d, dtype));
        if (rc != LA_OK) return rc;
    }
    // 2. exclusive prefixes in place (+ carry), total -> carry.  Without a
    // carry, the bf16 scan at 64 channels on chip (d = 32, 64) forms each
    // chunk's prefix from the partials itself, in the same order, and this
    // launch is not needed (720p-5s: 6 us of the call).
    const bool raw = !S_carry && dtype == LA_BF16 && d <= 64;
    if (!raw) {
        PrefixArgs pa;
        pa.partial = partial;
        pa.S_carry = S_carry;
        pa.z_carry = z_carry;
        pa.S_out = S_carry;
        pa.z_out = z_carry;
        pa.P = ps.P;
        rc = launch_kernel<PrefixArgs>(prefix_kernel(d), dim3((d * d + d + 255) / 256, g.BH), 0, st, pa);
        if (rc != LA_OK) return rc;
    }
    // 3. causal scan of every chunk from its prefix
    CausalArgs ca;
    ca.Q = Q;
    ca.K = K;
    ca.V = V;
    ca.O = O;
    ca.pre = partial;
    ca.raw_prefix = raw ? 1 : 0;
    ca.eps = eps;
    ca.chunk = pc.chunk;
    ca.P = pc.P;
    ca.g = g;
    return launch_kernel<CausalArgs>(causal_kernel(d, dtype, g.rope), dim3(pc.P * g.BH), pc.lds, st, ca, 256);
}

size_t elem_bytes(int dtype) { return dtype == LA_BF16 ? 2 : 4; }

// Plans depend only on sizes, so a plan failure is reported before any launch.
// *partials: the state plan's partial count (0 without a state pass).
int precheck_plans(int B, int H, int ntok, int n_offset, int d, int gt, int gh, int gw, int dtype,
                   bool state, bool apply, int* partials = nullptr) {
    const LaGeom g = make_geom(B, H, ntok, n_offset, d, gt, gh, gw);
    Plan pl;
    if (partials) *partials = 0;
    if (state) {
        int rc = plan_state(g, d, dtype, &pl);
        if (rc != LA_OK) return rc;
        if (partials) *partials = pl.P;
    }
    if (apply && ntok > 0) {
        ApplyPlan pa;
        int rc = plan_apply(g, d, dtype, &pa);
        if (rc != LA_OK) return rc;
    }
    return LA_OK;
}

// Largest partial count any call of these sizes plans (state pass in either
// dtype, token-causal pass): plans only grow with the token count, so this
// covers every block of a block-causal sequence of N tokens too.
int max_partials(int B, int H, int N, int d, int gt, int gh, int gw) {
    int P = 1;
    for (int dtype : {LA_BF16, LA_FP32}) {
        const LaGeom g = make_geom(B, H, N, 0, d, gt, gh, gw);
        Plan pl;
        if (plan_state(g, d, dtype, &pl) == LA_OK && pl.P > P) P = pl.P;
    }
    {
        const LaGeom g = make_geom(B, H, N > 0 ? N : 1, 0, d, gt, gh, gw);
        Plan pc;
        for (int dtype : {LA_BF16, LA_FP32})
            if (plan_causal(g, d, dtype, &pc) == LA_OK && pc.P > P) P = pc.P;
    }
    return P;
}

// Argument checks of the state pass shared by la_state_reduce and its
// no-allocation variant; *need = workspace bytes of the call's plan.
int state_reduce_checks(const void* K, const void* V, const float* S, const float* z, int B, int H, int N, int d,
                        int gt, int gh, int gw, float eps, int dtype, size_t* need) {
    int rc = check_common(B, H, N, d, gt, gh, gw, eps, dtype);
    if (rc != LA_OK) return rc;
    if (!S || !z || (N > 0 && (!K || !V))) return LA_E_NULLPTR;
    if (!aligned16(K) || !aligned16(V) || !aligned16(S) || !aligned16(z)) return LA_E_ALIGN;
    int partials = 0;
    rc = precheck_plans(B, H, N, 0, d, gt, gh, gw, dtype, true, false, &partials);
    if (rc != LA_OK) return rc;
    *need = ws_layout(B * H, d, partials).total;
    const size_t nS = (size_t)B * H * d * d * 4, nz = (size_t)B * H * d * 4;
    const size_t nkv = (size_t)B * H * N * d * elem_bytes(dtype);
    if (overlaps(S, nS, K, nkv) || overlaps(S, nS, V, nkv) || overlaps(z, nz, K, nkv) ||
        overlaps(z, nz, V, nkv) || overlaps(S, nS, z, nz))
        return LA_E_ALIAS;
    return LA_OK;
}

// Device address of the static scratch on the current device, looked up once
// per device (each device holds its own copy of the array at its own
// address).  The first call on a device also clears the counter region, on
// the caller's stream ahead of the caller's own work.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(hipStream_t st, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return LA_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        const size_t n16 = (size_t)kTicketHeads * 8 / 16;
        (void)hipGetLastError();
        hipLaunchKernelGGL(la_zero_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st, (u32x4*)ptr,
                           n16);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "la_zero_kernel launch");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LA_OK;
}

}  // namespace

extern "C" {

size_t la_workspace_bytes(int B, int H, int N, int d) {
    if (check_common(B, H, N, d, 0, 0, 0, 0.0f, LA_BF16) != LA_OK) return 0;
    return ws_layout(B * H, d, max_partials(B, H, N, d, 0, 0, 0)).total;
}

size_t la_workspace_bytes_grid(int B, int H, int N, int d, int gt, int gh, int gw) {
    if (check_common(B, H, N, d, gt, gh, gw, 0.0f, LA_BF16) != LA_OK) return 0;
    const int P0 = max_partials(B, H, N, d, 0, 0, 0);
    const int P1 = max_partials(B, H, N, d, gt, gh, gw);
    return ws_layout(B * H, d, P0 > P1 ? P0 : P1).total;
}

int la_state_reduce(const void* Q, const void* K, const void* V, void* O, float* S, float* z, void* ws,
                    size_t ws_bytes, int B, int H, int N, int d, int gt, int gh, int gw, int block_tokens,
                    float eps, int dtype, void* stream) {
    (void)Q;
    (void)O;
    (void)block_tokens;
    size_t need = 0;
    int rc = state_reduce_checks(K, V, S, z, B, H, N, d, gt, gh, gw, eps, dtype, &need);
    if (rc != LA_OK) return rc;
    if (!ws) return LA_E_NULLPTR;
    if (!aligned16(ws)) return LA_E_ALIGN;
    if (ws_bytes < need) return LA_E_WORKSPACE;
    const size_t nS = (size_t)B * H * d * d * 4, nz = (size_t)B * H * d * 4;
    const size_t nkv = (size_t)B * H * N * d * elem_bytes(dtype);
    if (overlaps(ws, ws_bytes, K, nkv) || overlaps(ws, ws_bytes, V, nkv) || overlaps(ws, ws_bytes, S, nS) ||
        overlaps(ws, ws_bytes, z, nz))
        return LA_E_ALIAS;
    return run_state(K, V, S, z, nullptr, nullptr, nullptr, nullptr, ws, B, H, N, 0, d, gt, gh, gw, dtype,
                     (hipStream_t)stream);
}

int la_state_reduce_noalloc(const void* Q, const void* K, const void* V, void* O, float* S, float* z, int B,
                            int H, int N, int d, int gt, int gh, int gw, int block_tokens, float eps, int dtype,
                            void* stream) {
    (void)Q;
    (void)O;
    (void)block_tokens;
    size_t need = 0;
    int rc = state_reduce_checks(K, V, S, z, B, H, N, d, gt, gh, gw, eps, dtype, &need);
    if (rc != LA_OK) return rc;
    if (need > LA_NOALLOC_SCRATCH_BYTES) {
        snprintf(g_hip_msg, sizeof(g_hip_msg),
                 "la_state_reduce_noalloc: these sizes need %zu bytes of scratch, the static scratch holds %zu",
                 need, (size_t)LA_NOALLOC_SCRATCH_BYTES);
        return LA_E_WORKSPACE;
    }
    void* ws = nullptr;
    rc = scratch_of_current_device((hipStream_t)stream, &ws);
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
    const size_t nS = (size_t)B * H * d * d * 4, nz = (size_t)B * H * d * 4;
    if (overlaps(O, nqo, Q, nqo) || overlaps(O, nqo, S, nS) || overlaps(O, nqo, z, nz))
        return LA_E_ALIAS;
    rc = precheck_plans(B, H, N, 0, d, gt, gh, gw, dtype, false, true);
    if (rc != LA_OK) return rc;
    return run_apply(Q, O, S, z, B, H, N, 0, d, gt, gh, gw, eps, dtype, (hipStream_t)stream);
}

size_t la_cross_workspace_bytes(int B, int H, int N_kv, int d) {
    if (check_common(B, H, N_kv, d, 0, 0, 0, 0.0f, LA_BF16) != LA_OK) return 0;
    return cross_ws_bytes(B * H, d, max_partials(B, H, N_kv, d, 0, 0, 0));
}

int la_cross_attention(const void* Q, const void* K, const void* V, void* O, void* ws, size_t ws_bytes, int B,
                       int H, int N_q, int N_kv, int d, float eps, int dtype, void* stream) {
    int rc = check_common(B, H, N_q, d, 0, 0, 0, eps, dtype);
    if (rc != LA_OK) return rc;
    rc = check_common(B, H, N_kv, d, 0, 0, 0, eps, dtype);
    if (rc != LA_OK) return rc;
    if (N_q == 0) return LA_OK;  // nothing to write
    if (!Q || !O || !ws || (N_kv > 0 && (!K || !V))) return LA_E_NULLPTR;
    if (!aligned16(Q) || !aligned16(O) || !aligned16(K) || !aligned16(V) || !aligned16(ws)) return LA_E_ALIGN;
    int partials = 0;
    rc = precheck_plans(B, H, N_kv, 0, d, 0, 0, 0, dtype, true, false, &partials);
    if (rc != LA_OK) return rc;
    rc = precheck_plans(B, H, N_q, 0, d, 0, 0, 0, dtype, false, true);
    if (rc != LA_OK) return rc;
    if (ws_bytes < cross_ws_bytes(B * H, d, partials)) return LA_E_WORKSPACE;
    const size_t nq = (size_t)B * H * N_q * d * elem_bytes(dtype);
    const size_t nkv = (size_t)B * H * N_kv * d * elem_bytes(dtype);
    if (overlaps(O, nq, Q, nq) || overlaps(O, nq, K, nkv) || overlaps(O, nq, V, nkv) || overlaps(ws, ws_bytes, Q, nq) ||
        overlaps(ws, ws_bytes, O, nq) || overlaps(ws, ws_bytes, K, nkv) || overlaps(ws, ws_bytes, V, nkv))
        return LA_E_ALIAS;
    const hipStream_t st = (hipStream_t)stream;
    if (dtype == LA_BF16 && d == 64 && N_kv <= KV_MAXKV && knob(K_CROSS_FUSED, 1) != 0) {
        rc = run_cross_fused(Q, K, V, O, B, H, N_q, N_kv, eps, st);
        if (rc != LA_E_UNSUPPORTED) return rc;
    }
    // two launches: the state pass into the workspace's S and z, then the apply
    const size_t off_S = align_up(ws_layout(B * H, d, partials).total, 256);
    float* S = (float*)((char*)ws + off_S);
    float* z = (float*)((char*)ws + off_S + align_up((size_t)B * H * d * d * 4, 256));
    rc = run_state(K, V, S, z, nullptr, nullptr, nullptr, nullptr, ws, B, H, N_kv, 0, d, 0, 0, 0, dtype, st);
    if (rc != LA_OK) return rc;
    return run_apply(Q, O, S, z, B, H, N_q, 0, d, 0, 0, 0, eps, dtype, st);
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
    int partials = 0;
    rc = precheck_plans(B, H, Lb, (int)start, d, gt, gh, gw, dtype, true, true, &partials);
    if (rc != LA_OK) return rc;
    const WsLayout L = ws_layout(B * H, d, partials);
    if (ws_bytes < L.total) return LA_E_WORKSPACE;
    const size_t nb = (size_t)B * H * Lb * d * elem_bytes(dtype);
    const size_t nS = (size_t)B * H * d * d * 4, nz = (size_t)B * H * d * 4;
    if (overlaps(O, nb, Q, nb) || overlaps(O, nb, K, nb) || overlaps(O, nb, V, nb) ||
        overlaps(O, nb, S_carry, nS) || overlaps(O, nb, z_carry, nz) || overlaps(S_carry, nS, z_carry, nz) ||
        overlaps(S_carry, nS, K, nb) || overlaps(S_carry, nS, V, nb) || overlaps(z_carry, nz, K, nb) ||
        overlaps(z_carry, nz, V, nb) || overlaps(ws, ws_bytes, S_carry, nS) || overlaps(ws, ws_bytes, z_carry, nz) ||
        overlaps(ws, ws_bytes, O, nb) || overlaps(ws, ws_bytes, Q, nb) || overlaps(ws, ws_bytes, K, nb) ||
        overlaps(ws, ws_bytes, V, nb))
        return LA_E_ALIAS;
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
    if ((S_carry == nullptr) != (z_carry == nullptr)) return LA_E_NULLPTR;
    if (!ws || (N > 0 && (!Q || !K || !V || !O))) return LA_E_NULLPTR;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(ws) ||
        !aligned16(S_carry) || !aligned16(z_carry))
        return LA_E_ALIGN;
    if (N == 0) return ws_bytes < ws_layout(B * H, d, 1).total ? LA_E_WORKSPACE : LA_OK;  // the carry stays
    Plan pc, ps;
    {
        const LaGeom g = make_geom(B, H, N, n_offset, d, gt, gh, gw);
        rc = plan_causal(g, d, dtype, &pc);
        if (rc != LA_OK) return rc;
        rc = plan_state(g, d, dtype, &ps, pc.chunk, tc_half_state(d, dtype) ? StateBf16Cfg<64, 512>::SMEM_FIXED : 0);
        if (rc != LA_OK) return rc;
    }
    if (ws_bytes < ws_layout(B * H, d, ps.P).total) return LA_E_WORKSPACE;
    const size_t nb = (size_t)B * H * N * d * elem_bytes(dtype);
    const size_t nS = S_carry ? (size_t)B * H * d * d * 4 : 0, nz = z_carry ? (size_t)B * H * d * 4 : 0;
    if (overlaps(O, nb, Q, nb) || overlaps(O, nb, K, nb) || overlaps(O, nb, V, nb) ||
        overlaps(O, nb, S_carry, nS) || overlaps(O, nb, z_carry, nz) || overlaps(S_carry, nS, z_carry, nz) ||
        overlaps(S_carry, nS, K, nb) || overlaps(S_carry, nS, V, nb) || overlaps(S_carry, nS, Q, nb) ||
        overlaps(z_carry, nz, K, nb) || overlaps(z_carry, nz, V, nb) || overlaps(z_carry, nz, Q, nb) ||
        overlaps(ws, ws_bytes, S_carry, nS) || overlaps(ws, ws_bytes, z_carry, nz) ||
        overlaps(ws, ws_bytes, O, nb) || overlaps(ws, ws_bytes, Q, nb) || overlaps(ws, ws_bytes, K, nb) ||
        overlaps(ws, ws_bytes, V, nb))
        return LA_E_ALIAS;
    return run_token_causal(Q, K, V, O, S_carry, z_carry, ws, B, H, N, n_offset, d, gt, gh, gw, eps, dtype,
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
    a.gm = knob(K_TCONV_GM, 8);
    a.gn = knob(K_TCONV_GN, 7);
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

int la_set_tuning(const char* name, int value) {
    if (!name) return LA_E_NULLPTR;
    for (int k = 0; k < K_COUNT; ++k) {
        if (strcmp(name, kKnobs[k].name) != 0) continue;
        if (value < 0) {
            g_knob[k] = -1;
            return LA_OK;
        }
        if (value < kKnobs[k].lo || value > kKnobs[k].hi) return LA_E_SHAPE;
        if (k == K_TC_STATE_THREADS && value != 512 && value != 1024) return LA_E_SHAPE;
        g_knob[k] = value;
        return LA_OK;
    }
    return LA_E_UNSUPPORTED;
}

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
