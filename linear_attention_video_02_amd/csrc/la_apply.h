// Apply pass of ReLU linear attention (numerator / denominator of Eq. 2 on the
// SANA-Video analysis page, section 3.4 "Integration of 3D RoPE"):
//
//   O_i = RoPE(relu(Q_i)) S / (relu(Q_i) . z + eps)
//
// One HBM read of Q and one write of O; S and z (a few KB per head) come from
// L2.  Rows with relu(Q_i) = 0 produce exact zeros.
#pragma once

#include "la_common.h"
#include "la_state.h"

struct ApplyArgs {
    const void* Q;
    void* O;
    const float* S;  // [BH][D*D]
    const float* z;  // [BH][D]
    // cross-attention in one launch (the KV instance): S and z of each head
    // formed in the prologue from its nkv keys/values instead of read
    const void* K;   // [BH][nkv][D]
    const void* V;
    int nkv;
    float eps;
    int chunk;       // ilv = 0: tokens per workgroup
    int P;           // workgroups per head
    int ilv;         // bf16: 1 = the head's P workgroups take interleaved units of the whole head
    int nph;         // ilv = 1: heads per workgroup, one after another (phases)
    int hs;          // ilv = 1: head slots; phase k of slot j is head k * hs + j
    int spread;      // ilv = 1: a slot's workgroups lie on all 8 XCDs (P % 8 == 0)
    LaGeom g;
};

// ---------------------------------------------------------------------------
// bf16: MFMA with C = S^T . RoPE(relu Q)^T, so that every accumulator a lane
// holds belongs to one token (column n = lane % 16) and the B operand -- 8
// consecutive channels of one token -- is a plain 16-byte load of Q.
// Numerator: v_mfma_f32_16x16x32_f16 on fp16 operands.  S^T is scaled by a
// power of two per head (its largest entry to [2^13, 2^14)) and rounded to
// fp16; RoPE(relu Q) is rounded to fp16 as it is (fp16's 11-bit significand
// makes one product per k-step as accurate as three bf16 hi/lo products --
// a single bf16 rounding of either factor costs up to ~1% in rows whose sum
// over channels cancels).  A group of 16 tokens whose relu(Q) values are
// not all within [2^-6, 2^14) (or zero) -- where fp16 could overflow or lose
// precision -- is scaled by a power of two per token first; powers of two
// are exact and are undone after the sum.  Denominator: un-rotated relu(Q),
// exact in bf16, against z (bf16 hi + lo on the MFMA at d <= 64, fp32 FMA
// at d >= 112).
//
// Lane (n = lane % 16, g = lane / 16) handles token n of a 16-token group and
// the key channels 32*ks + 8*g .. +7, ks = 0 .. d/32 - 1.  Output tile T (16
// value channels) row 4g+i maps to value channel 32*(T/2) + 8g + 4*(T%2) + i,
// so a lane ends with 8 consecutive output channels per pair of tiles: one
// 16-byte store each.  The denominator is summed over the 4 lanes of a token
// with two cross-lane xors.
//
// Work split (interleaved mode, the default).  Few heads are in flight at a
// time: P workgroups share each head (unit u of the head goes to workgroup
// u mod P), and every workgroup works through nph heads one after another
// (phase k of head slot j is head k * hs + j).  A copy of Q to O shaped like
// this runs at the rate of a plain copy when a handful of heads are in
// flight, and ~10% slower when every head of the call is (one read and one
// write window per head).  Each head of the workgroup has an LDS operand
// buffer (S^T in fp16, scaled, and z).  Phase 0's is converted by every wave
// before the start, while the first units of Q are in flight; wave w
// converts phase w + 1's after its first unit (or before it would first
// wait), so the start does not wait for every head's S.  A wave that moves on
// to the next head reloads its operands from that head's buffer.  Each wave
// takes UNIT-token units from the workgroup's LDS queue of the current phase
// and keeps DEPTH units of Q in flight.
// ---------------------------------------------------------------------------
template <int D>
struct ApplyBf16Cfg {
    static constexpr int DP = Pad<D>::P;  // channels on chip (zero above D)
    // d <= 64: 8 waves per CU (2 per SIMD: S^T hi + lo in registers);
    // d >= 112: 12 waves (S^T read from LDS per k-step, <= 168 registers a lane)
    static constexpr int THREADS = D <= 64 ? 512 : 768;
    static constexpr int NW = THREADS / 64;
    static constexpr int KS = DP / 32;  // 32-channel k-steps
    static constexpr int NT = DP / 16;  // 16-channel output tiles
    static constexpr int GR = D <= 64 ? 2 : 1;   // 16-token groups per unit of work
    static constexpr int UNIT = 16 * GR;         // tokens a wave takes from the queue at a time
    static constexpr int DEPTH = D <= 64 ? 3 : 2;  // units of Q in flight per wave
    // d >= 112: the MFMA A fragments are read from the LDS copy of S^T per
    // k-step (128 x 128 fp16 in registers would take 128 a lane)
    static constexpr bool SLDS = DP > 64;
    // d = 112: the last k-step covers channels 96..111 only, on the K = 16
    // MFMA (v_mfma_f32_16x16x16_f16): no work and no LDS reads on the key
    // channels 112..127, so the S^T copy needs no zeroed padding columns.
    // (Its rows 112..127 -- value channels past d -- feed only outputs that
    // are never stored.)
    static constexpr bool HALF = D == 112;
    // heads per workgroup at most (their S^T copies share the LDS)
    static constexpr int MAXPH = DP > 64 ? 2 : 8;
    // d = 64: Q and O pass through a per-wave LDS tile so that every global
    // load / store instruction moves 8 whole 128-byte rows (the MFMA operand
    // layout would touch 16 rows per instruction, half of each line).
    static constexpr bool STG = D == 64;
    static constexpr int RPI = 8;                          // rows per staged load / store
    static constexpr int NI = UNIT / RPI;                  // staged loads per unit (= GR * KS)
    // d >= 112: a 16-token unit of Q (or O) is one contiguous block of UB
    // bytes, moved by NIW instructions of 16 bytes a lane (1 KB each) through
    // a per-wave LDS tile of UNIT rows x DP channels (the MFMA operand layout
    // would touch 16 rows per instruction, 64 bytes of each, and at d = 112
    // those pieces straddle 128-byte lines).  Lanes past the unit's end (the
    // last 512 bytes of the fourth instruction at d = 112) load and store out
    // of range and park in the tile's padding chunks.
    static constexpr bool STW = D >= 112;
    static constexpr int UB = UNIT * D * 2;
    static constexpr int NIW = (UB + 1023) / 1024;
    static constexpr int STGBYTES = STG ? NW * 2 * UNIT * D * 2 : STW ? NW * UNIT * DP * 2 : 0;
    static constexpr int SHEAD = DP * DP * 2;              // fp16 S^T of one head
    static constexpr int ZHEAD = DP * 4;                   // z of one head (zero above d)
    // LDS: staging tiles, then nph x (S^T, z), then the RoPE table
    static constexpr int FIXED = STGBYTES;
    static constexpr int PERHEAD = SHEAD + ZHEAD;
    static_assert(!STG || NI == GR * KS, "staged unit = register ring slot");
    static_assert(!STW || (GR == 1 && NIW == KS), "whole-unit staging = register ring slot");
    static_assert(!STW || (NIW * 1024 - UB) / 16 <= UNIT * (DP - D) / 8, "parking slots");
};

// Element offset of row r, 16-byte chunk c of a wave's staging tile
// ([UNIT][64] bf16): chunk c of row r sits at c ^ f(r), which keeps both the
// row-major 8-rows-per-instruction accesses and the MFMA-layout accesses
// (16 consecutive rows at one chunk) free of bank conflicts.
__device__ __forceinline__ int stg_off(int r, int c) {
    return r * 64 + ((c ^ ((r ^ (r >> 3)) & 7)) << 3);
}

// Element offset of row r (< 16), 16-byte chunk c of a wave's whole-unit tile
// ([16][DP] bf16, d >= 112): chunk c of row r sits at c ^ r, so the 16 rows
// read at one chunk (MFMA operand layout) cover all banks once.
template <int DP>
__device__ __forceinline__ int stw_off(int r, int c) {
    return r * DP + ((c ^ r) << 3);
}

// Element offset of S^T row pr (= 16 T + m, see below), 16-byte chunk c, in
// the LDS copy: chunks are XOR-swizzled by row (within the row's DP / 8
// chunks) so that consecutive rows read at one chunk spread over the banks.
template <int DP>
__device__ __forceinline__ int st_off(int pr, int c) {
    return pr * DP + ((c ^ (pr & (DP / 8 - 1))) << 3);
}

// Row of the S^T copy that holds value channel co: the MFMA output tile T
// and row m within it (value channel 32 (T/2) + 8 (m/4) + 4 (T%2) + m%4).
__device__ __forceinline__ int st_row(int co) {
    const int T = 2 * (co >> 5) + ((co >> 2) & 1);
    const int m = (((co >> 3) & 3) << 2) | (co & 3);
    return 16 * T + m;
}

// Which slot and position the workgroup takes.  With `spread` the P
// workgroups of a slot lie on all 8 XCDs (workgroup i runs on XCD i % 8);
// otherwise on as few as possible (whole heads per XCD).
__device__ __forceinline__ void apply_item_of_block(int P, int NS, int spread, int& slot, int& p) {
    const int i = blockIdx.x;
    if (spread) {
        const int q = i >> 3;
        slot = q % NS;
        p = (q / NS) * 8 + (i & 7);
        return;
    }
    const int T = P * NS;
    const int k = (T % 8 == 0) ? (i % 8) * (T / 8) + i / 8 : i;
    slot = k / P;
    p = k % P;
}

// NPH: register slots for S, at least the heads per workgroup (a.nph)
// KV: cross-attention in one launch, S and z formed from K and V (d = 64, no
// RoPE, at most KV_MAXKV keys/values a head; the instance with NPH slots runs
// with exactly NPH heads a workgroup)
constexpr int KV_MAXKV = 512;
template <int D, bool ROPE, int NPH, bool KV = false>
__global__ __launch_bounds__(ApplyBf16Cfg<D>::THREADS) void la_apply_bf16_kernel(ApplyArgs a) {
    using C = ApplyBf16Cfg<D>;
    static_assert(!KV || (D == 64 && !ROPE && C::STGBYTES == 64 * 1024), "one-launch cross-attention layout");
    extern __shared__ __align__(16) unsigned char smem[];
    const bool ilv = a.ilv != 0;
    const int nph = ilv ? a.nph : 1;
    uint16_t* stg = (uint16_t*)smem;                                // [NW][Q, O][UNIT][D] (d = 64)
    uint16_t* st16 = (uint16_t*)(smem + C::FIXED);                  // [nph][DP*DP] fp16 S^T
    float* zs = (float*)(smem + C::FIXED + nph * C::SHEAD);         // [nph][DP] z
    float2* tab = (float2*)(smem + C::FIXED + nph * C::PERHEAD);
    __shared__ int q_next[NPH];         // next unit of each phase's queue, in tokens
    __shared__ float smax[NPH][C::NW];  // per-wave max |S| of each head
    __shared__ int eSs[NPH];            // per-head exponent of the S^T scale

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int BH = a.g.BH;
    int slot, p;
    apply_item_of_block(a.P, ilv ? a.hs : BH, ilv ? a.spread : 0, slot, p);
    auto head_of = [&](int ph) -> int { return ilv ? ph * a.hs + slot : slot; };
    const int ntok = a.g.ntok;
    const int c0 = ilv ? 0 : p * a.chunk;
    const int c1 = ilv ? ntok : min(c0 + a.chunk, ntok);
    const int len = c1 > c0 ? c1 - c0 : 0;
    // queue position q (in tokens) -> first token of the unit, within [c0, c1)
    auto tok_of = [&](int q) -> int { return ilv ? ((q / C::UNIT) * a.P + p) * C::UNIT : q; };
    // Q and O of a head's chunk through descriptors bounded to [c0, c1): rows
    // past c1 read as zeros and their stores are dropped.
    const uint32_t chunk_bytes = (uint32_t)len * D * 2;
    // (the head index goes through readfirstlane: the compiler cannot prove
    // it wave-uniform once it comes out of the phase queues, and a
    // descriptor it takes for divergent gets every load and store wrapped in
    // a loop over lanes)
    auto q_rsrc = [&](int head) {
        head = __builtin_amdgcn_readfirstlane(head);
        return make_rsrc((const uint16_t*)a.Q + ((size_t)head * ntok + c0) * D, chunk_bytes);
    };
    auto o_rsrc = [&](int head) {
        head = __builtin_amdgcn_readfirstlane(head);
        return make_rsrc((uint16_t*)a.O + ((size_t)head * ntok + c0) * D, chunk_bytes);
    };

    if (threadIdx.x < NPH) q_next[threadIdx.x] = threadIdx.x == 0 ? C::NW * C::DEPTH * C::UNIT : 0;

    // S of every head of this workgroup: phase 0's before the first Q loads,
    // the others after them.  Loads return in order: phase 0's conversion
    // then waits for its own S only, and the first units of Q do not queue
    // behind every head's S.  Every register slot loads (a phase past nph
    // reloads phase 0's head) so that the compiler counts the loads exactly.
    // A thread takes column segments of S: segment g is value channel
    // co = g % D, key channels 8 kb .. 8 kb + 7 (kb = g / D), read as 8 words
    // that consecutive lanes take from consecutive channels of a row (256
    // bytes a wave instruction).  Rounded to fp16, a segment is one 16-byte
    // piece of a row of S^T in LDS, where each lane reads its fragments (as
    // 2-byte pieces, the transposed writes took 1.7 us of the SANA-2B apply).
    constexpr int NSEG = D * (D / 8);
    constexpr int SC = (NSEG + C::THREADS - 1) / C::THREADS;  // segments a thread per head
    float scol[NPH][SC][8];
    auto seg_at = [&](int i) { return (int)threadIdx.x + i * C::THREADS; };
    auto seg_off = [&](int sg) {  // float offset of the segment's first entry (0 past the end)
        return sg < NSEG ? 8 * (sg / D) * D + sg % D : 0;
    };
    auto load_s = [&](int ph) {
        const float* Sh = a.S + (size_t)head_of(ph < nph ? ph : 0) * D * D;
#pragma unroll
        for (int i = 0; i < SC; ++i) {
            const int o = seg_off(seg_at(i));
#pragma unroll
            for (int r = 0; r < 8; ++r) scol[ph][i][r] = Sh[o + r * D];
        }
    };
    // KV instance: every load of a head's keys/values at once (at most 512
    // tokens: two fills of 256 tokens, 16-byte pieces: thread -> rows
    // 64 j + sr of a fill, channels 8 sc .. 8 sc + 7), phase 0's ahead of the
    // first units of Q, the next phase's as soon as this one's are staged;
    // rows past nkv read as zeros (no traffic)
    u32x4 kvk[KV ? 2 : 1][4], kvv[KV ? 2 : 1][4];
    const int kv_sr = threadIdx.x >> 3, kv_sc = threadIdx.x & 7;
    const uint32_t kv_bytes = KV ? (uint32_t)a.nkv * D * 2 : 0u;
    auto kv_issue = [&](int ph) {
        const int hd = __builtin_amdgcn_readfirstlane(head_of(ph < nph ? ph : 0));
        const BufRsrc Kr = make_rsrc((const uint16_t*)a.K + (size_t)hd * a.nkv * D, kv_bytes);
        const BufRsrc Vr = make_rsrc((const uint16_t*)a.V + (size_t)hd * a.nkv * D, kv_bytes);
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t off = (uint32_t)((256 * f + 64 * j + kv_sr) * D + 8 * kv_sc) * 2u;
                kvk[f][j] = buf_load16(Kr, off);
                kvv[f][j] = buf_load16(Vr, off);
            }
    };
    if constexpr (KV) {
        kv_issue(0);
    } else {
        load_s(0);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of Q's

    // the ring: slot s holds the unit (phase, first token) whose Q is in qr[s]
    int wph = 0;  // this wave's current phase for taking units
    auto take = [&]() -> int2 {
        for (;;) {
            if (wph >= nph) return make_int2(nph, 0);
            int v = 0;
            if (lane == 0) v = atomicAdd(&q_next[wph], C::UNIT);
            const int tok = tok_of(__builtin_amdgcn_readfirstlane(v));
            if (tok < len && head_of(wph) < BH) return make_int2(wph, tok);
            ++wph;
        }
    };
    // whole-unit staging: each lane's tile slot for staged instruction i
    int woff[C::STW ? C::NIW : 1];
    bool wok[C::STW ? C::NIW : 1];
    if (C::STW) {
#pragma unroll
        for (int i = 0; i < C::NIW; ++i) {
            const int b = 1024 * i + 16 * lane;
            wok[i] = b < C::UB;
            if (wok[i]) {
                woff[i] = stw_off<C::DP>(b / (2 * D), (b % (2 * D)) / 16);
            } else {  // a padding chunk (channel >= d) of some row (d < DP only)
                constexpr int pads = C::DP > D ? (C::DP - D) / 8 : 1;
                const int k = (b - C::UB) / 16;
                woff[i] = stw_off<C::DP>(k / pads, D / 8 + k % pads);
            }
        }
    }
    u32x4 qr[C::DEPTH][C::GR][C::KS];
    auto load_unit = [&](u32x4 (&q)[C::GR][C::KS], int2 u) {
        const BufRsrc Qr = q_rsrc(u.x < nph ? head_of(u.x) : slot);
        const int u0 = u.x < nph ? u.y : len;  // none: a read past the end (zeros)
        if (C::STW) {  // byte 1024 i + 16 lane of the unit (past the unit: out of range, zeros)
#pragma unroll
            for (int i = 0; i < C::NIW; ++i)
                q[0][i] = buf_load16(Qr, wok[i] ? (uint32_t)u0 * (2u * D) + (uint32_t)(1024 * i + 16 * lane) : chunk_bytes);
            return;
        }
        if (C::STG) {  // whole rows: lane -> row RPI*i + lane/8, 16-byte chunk lane%8
#pragma unroll
            for (int i = 0; i < C::NI; ++i)
                q[i / C::KS][i % C::KS] =
                    buf_load16(Qr, (uint32_t)((u0 + C::RPI * i + (lane >> 3)) * D + 8 * (lane & 7)) * 2u);
            return;
        }
#pragma unroll
        for (int r = 0; r < C::GR; ++r) {
            const int tl = u0 + 16 * r + n;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                if (C::HALF && ks == C::KS - 1) {  // channels 32 ks + 4 g .. +3
                    const u32x2v h = buf_load8(Qr, (uint32_t)(tl * D + 32 * ks + 4 * g) * 2u);
                    q[r][ks] = u32x4{h[0], h[1], 0u, 0u};
                } else {
                    q[r][ks] = buf_load16(Qr, (uint32_t)(tl * D + 32 * ks + 8 * g) * 2u);
                }
            }
        }
    };
    // first DEPTH units of each wave: fixed positions of phase 0's queue (the
    // queue starts past them), so their loads go out before the prologue work.
    // A position past the head's end (tiny heads) leaves the slot to be
    // filled from the queues once they are initialised (x = -1).
    int2 us[C::DEPTH];
    bool fixed = head_of(0) < BH;
#pragma unroll
    for (int s = 0; s < C::DEPTH; ++s) {
        const int tok = tok_of((s * C::NW + wave) * C::UNIT);
        fixed = fixed && tok < len;  // (tokens grow with s: once past the end, all later are too)
        us[s] = fixed ? make_int2(0, tok) : make_int2(-1, 0);
        // (unconditional, a pending slot reading past the end: with every
        // load issued the compiler can count them exactly)
        load_unit(qr[s], fixed ? us[s] : make_int2(nph, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!KV) {
#pragma unroll
        for (int ph = 1; ph < NPH; ++ph) load_s(ph);
    } else {
        // S = relu(K)^T V on v_mfma_f32_32x32x16_bf16 (relu K and V exact in
        // bf16, every product exact in fp32): wave w sums the 32 x 32 tile
        // (w & 1, (w >> 1) & 1) over token half w >> 2 of each fill, the
        // halves are added in LDS, and the rows of S go to the registers the
        // conversion below reads (as if loaded from S).  z: per-thread sums
        // of relu(K), then across the lanes and waves.  The Q/O staging tiles
        // are free until the unit loop: during a fill relu K [0, 32 KB) and
        // V [32, 64 KB); then the upper halves' tiles [0, 16 KB), S rows
        // [16, 32 KB), per-wave z [32, 34 KB).
        uint16_t* kt = stg;
        uint16_t* vt = stg + 256 * 64;
        float* red = (float*)smem;
        float* srw = (float*)(smem + 16384);
        float* zw = (float*)(smem + 32768);
        const int i16 = lane & 15, q2 = (lane >> 4) & 1, gq = lane >> 5, m32 = lane & 31;
        const int rd_row = 8 * gq + (i16 >> 2), rd_col = 16 * q2 + 4 * (i16 & 3);
        const int tile = wave & 3, ci = tile & 1, cj = tile >> 1, th = wave >> 2;
        const int nfill = (a.nkv + 255) / 256;
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph) {
            float zp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) zp[e] = 0.0f;
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                if (f < nfill) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u32x4 w;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            w[i] = relu_bf16x2(kvk[f][j][i]);
                            zp[2 * i] += bf_lo(w[i]);
                            zp[2 * i + 1] += bf_hi(w[i]);
                        }
                        *(u32x4*)(kt + swz<64>(64 * j + kv_sr, 8 * kv_sc)) = w;
                        *(u32x4*)(vt + swz<64>(64 * j + kv_sr, 8 * kv_sc)) = kvv[f][j];
                    }
                    lds_barrier();
#pragma unroll
                    for (int st = 0; st < 8; ++st) {
                        const int r0 = 128 * th + 16 * st + rd_row, r1 = r0 + 4;
                        const bf16x8 A = lds_read_tr8(kt + swz<64>(r0, 32 * ci + rd_col),
                                                      kt + swz<64>(r1, 32 * ci + rd_col));
                        const bf16x8 B = lds_read_tr8(vt + swz<64>(r0, 32 * cj + rd_col),
                                                      vt + swz<64>(r1, 32 * cj + rd_col));
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc, 0, 0, 0);
                    }
                    lds_barrier();  // tiles free for the next fill
                }
            }
            // the next phase's keys/values (this phase's are all staged; every
            // phase of this instance is a head of the workgroup: nph = NPH)
            if (ph + 1 < NPH) kv_issue(ph + 1);
            if (th == 1) {
#pragma unroll
                for (int r = 0; r < 16; r += 4)
                    *(f32x4*)(red + ((tile * 4 + r / 4) * 64 + lane) * 4) =
                        f32x4{acc[r], acc[r + 1], acc[r + 2], acc[r + 3]};
            }
#pragma unroll
            for (int msk = 8; msk < 64; msk <<= 1)
#pragma unroll
                for (int e = 0; e < 8; ++e) zp[e] += __shfl_xor(zp[e], msk);
            if (lane < 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) zw[wave * 64 + 8 * lane + e] = zp[e];
            }
            lds_barrier();
            if (th == 0) {
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    const f32x4 u = *(const f32x4*)(red + ((tile * 4 + r / 4) * 64 + lane) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[r + e] += u[e];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    srw[(32 * ci + 8 * (r >> 2) + 4 * gq + (r & 3)) * 64 + 32 * cj + m32] = acc[r];
            }
            if (threadIdx.x < 64) {
                float zsum = 0.0f;
#pragma unroll
                for (int w = 0; w < C::NW; ++w) zsum += zw[w * 64 + threadIdx.x];
                zs[ph * C::DP + threadIdx.x] = zsum;
            }
            lds_barrier();
#pragma unroll
            for (int i = 0; i < SC; ++i) {
                const int o = seg_off(seg_at(i));  // (srw rows have D = 64 entries)
#pragma unroll
                for (int r = 0; r < 8; ++r) scol[ph][i][r] = srw[o + r * D];
            }
            lds_barrier();  // before the next head's tiles
        }
    }

    int t_lo = 0, nt = 1;
    Rope4 r4[C::KS];
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
        // pairs past d / 2 hold zeros: any table entry rotates them to zeros
        // (the half last k-step: pairs 16 ks + 2 g, + 1)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            r4[ks] = rope4_make(C::HALF && ks == C::KS - 1 ? 16 * ks + 2 * g
                                : (C::DP == D || 32 * ks + 8 * g < D) ? 16 * ks + 4 * g : 0, nt, a.g);
    }

    // each head's largest |S|: per thread, per wave, then over the waves
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        if (ph < nph && head_of(ph) < BH) {
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < SC; ++i) {
                if (seg_at(i) < NSEG)
#pragma unroll
                    for (int r = 0; r < 8; ++r) amax = fmaxf(amax, fabsf(scol[ph][i][r]));
            }
            amax = wave_max(amax);
            if (lane == 0) smax[ph][wave] = amax;
        }
    }
    lds_barrier();  // per-wave maxima (and the RoPE table) visible
    // eS: the head's largest |S| times 2^-eS lies in [2^13, 2^14); S^T rows in
    // the MFMA row order: row pr = 16 T + m holds value channel co(T, m),
    // element k is S[k][co] 2^-eS (zero past d)
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        const int hd = head_of(ph);
        if (ph < nph && hd < BH) {
            float hmax = 0.0f;
#pragma unroll
            for (int w = 0; w < C::NW; ++w) hmax = fmaxf(hmax, smax[ph][w]);
            int eS = 0;
            if (hmax > 0.0f) {
                (void)frexpf(hmax, &eS);
                eS -= 14;
            }
            if (threadIdx.x == 0) eSs[ph] = eS;
            uint16_t* sth = st16 + ph * C::DP * C::DP;
            auto put_st = [&](int k, int co, float sv) {
                sth[st_off<C::DP>(st_row(co), k >> 3) + (k & 7)] =
                    __builtin_bit_cast(uint16_t, (_Float16)ldexpf(sv, -eS));
            };
#pragma unroll
            for (int i = 0; i < SC; ++i) {
                const int sg = seg_at(i);
                if (sg < NSEG) {
                    u32x4 w;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const _Float16 lo = (_Float16)ldexpf(scol[ph][i][2 * r], -eS);
                        const _Float16 hi = (_Float16)ldexpf(scol[ph][i][2 * r + 1], -eS);
                        w[r] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                    }
                    *(u32x4*)(sth + st_off<C::DP>(st_row(sg % D), sg / D)) = w;
                }
            }
            // the padding rows and columns (key or value channel >= d); with the
            // half last k-step no padding entry is ever read into a stored output
            constexpr int padc = C::DP > D ? C::DP - D : 1;  // (the loop runs only where DP > d)
            for (int e = threadIdx.x; !C::HALF && e < C::DP * C::DP - D * D; e += C::THREADS) {
                int k, co;
                if (e < D * (C::DP - D)) {
                    k = e / padc;
                    co = D + e % padc;
                } else {
                    k = D + (e - D * (C::DP - D)) / C::DP;
                    co = (e - D * (C::DP - D)) % C::DP;
                }
                put_st(k, co, 0.0f);
            }
            for (int c = threadIdx.x; c < C::DP; c += C::THREADS)
                if (!KV) zs[ph * C::DP + c] = c < D ? a.z[(size_t)hd * D + c] : 0.0f;
        }
    }
    lds_barrier();  // S^T copies, z, exponents and the queue heads visible
#pragma unroll
    for (int s = 0; s < C::DEPTH; ++s)
        if (us[s].x < 0) {
            us[s] = take();
            load_unit(qr[s], us[s]);
        }

    // operands of the head in use: S^T fragments (d <= 64, registers) --
    // value channel co(T, n), key channels 32 ks + 8 g .. +7 -- and z; d <= 64
    // also holds z as an A tile of 16 identical rows (bf16 hi + lo) for the
    // denominator on the MFMA (the un-rotated relu(q), exact in bf16, is B)
    f16x8 A16[C::SLDS ? 1 : C::NT][C::KS];
    bf16x8 Azh[C::SLDS ? 1 : C::KS], Azl[C::SLDS ? 1 : C::KS];
    int cur = -1, eS = 0;
    const uint16_t* sth = st16;
    const float* zh = zs;
    auto use_head = [&](int ph) {
        cur = ph;
        eS = eSs[ph];
        sth = st16 + ph * C::DP * C::DP;
        zh = zs + ph * C::DP;
        if (!C::SLDS) {
#pragma unroll
            for (int T = 0; T < C::NT; ++T)
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks)
                    A16[T][ks] = *(const f16x8*)(sth + st_off<C::DP>(16 * T + n, 4 * ks + g));
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const f32x4 z0 = *(const f32x4*)(zh + 32 * ks + 8 * g);
                const f32x4 z1 = *(const f32x4*)(zh + 32 * ks + 8 * g + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float zv = e < 4 ? z0[e] : z1[e - 4];
                    const __bf16 hi = (__bf16)zv;
                    Azh[ks][e] = hi;
                    Azl[ks][e] = (__bf16)(zv - (float)hi);
                }
            }
        }
    };

    bool more = true;
    while (more) {
#pragma unroll
        for (int s = 0; s < C::DEPTH; ++s) {
            const int2 uc = us[s];
            if (uc.x >= nph) {  // units are taken in increasing order: nothing left
                more = false;
                break;
            }
            const int u0 = uc.y;
            if (uc.x != cur) use_head(uc.x);
            const BufRsrc Or = o_rsrc(head_of(uc.x));
            u32x4 qc[C::GR][C::KS];
            // this wave's Q tile, then its O tile (d >= 112: one tile, O over Q)
            uint16_t* wq = stg + wave * (C::STG ? 2 * C::UNIT * D : C::UNIT * C::DP);
            uint16_t* wo = C::STG ? wq + C::UNIT * D : wq;
            if (C::STW) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int i = 0; i < C::NIW; ++i) *(u32x4*)(wq + woff[i]) = qr[s][0][i];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    if (C::HALF && ks == C::KS - 1) {  // channels 32 ks + 4 g .. +3
                        const u32x2v h = *(const u32x2v*)(wq + stw_off<C::DP>(n, 4 * ks + (g >> 1)) + 4 * (g & 1));
                        qc[0][ks] = u32x4{h[0], h[1], 0u, 0u};
                    } else {
                        qc[0][ks] = *(const u32x4*)(wq + stw_off<C::DP>(n, 4 * ks + g));
                    }
                }
            } else if (C::STG) {
                // rows into LDS, then each lane reads its MFMA operand (token n, 8 channels)
#pragma unroll
                for (int i = 0; i < C::NI; ++i)
                    *(u32x4*)(wq + stg_off(C::RPI * i + (lane >> 3), lane & 7)) = qr[s][i / C::KS][i % C::KS];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int r = 0; r < C::GR; ++r)
#pragma unroll
                    for (int ks = 0; ks < C::KS; ++ks) qc[r][ks] = *(const u32x4*)(wq + stg_off(16 * r + n, 4 * ks + g));
            } else {
#pragma unroll
                for (int r = 0; r < C::GR; ++r)
#pragma unroll
                    for (int ks = 0; ks < C::KS; ++ks) qc[r][ks] = qr[s][r][ks];
            }
            us[s] = take();
            load_unit(qr[s], us[s]);

#pragma unroll
            for (int r = 0; r < C::GR; ++r) {
                const int tl = u0 + 16 * r + n;  // token within the chunk
                Pos3 ps;
                if (ROPE) ps = token_pos8((uint32_t)(a.g.n_offset + c0 + min(tl, len - 1)), t_lo, a.g);
                float den = 0.0f;
                f32x4 dacc = f32x4{0.f, 0.f, 0.f, 0.f};
                f32x4 acc[C::NT];
#pragma unroll
                for (int T = 0; T < C::NT; ++T) acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
                // relu(Q) of the group (channels past d, loaded from the next
                // row at d = 112, are zeroed): the token's largest value (0:
                // the row is zero and so is its output), and whether any lane
                // holds a value fp16 cannot carry exactly enough: then every
                // token of the group is scaled by 2^sc, sc = 13 - (exponent of
                // its largest relu(Q) value)
                uint32_t m16 = 0;
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    // (the half last k-step holds 4 live channels and 4 zeros)
                    const bool live = C::DP == D || (C::HALF && ks == C::KS - 1) || 32 * ks + 8 * g < D;
                    const uint32_t mk = live ? max_relu_bits8(qc[r][ks]) : 0u;
                    m16 = mk > m16 ? mk : m16;
                }
                uint32_t tm = m16;
                tm = max(tm, (uint32_t)__shfl_xor((int)tm, 16));
                tm = max(tm, (uint32_t)__shfl_xor((int)tm, 32));
                // bf16 bit patterns of 2^-6 and 2^14
                const bool odd = m16 != 0 && (m16 < 0x3C80u || m16 >= 0x4680u);
                // (d >= 112: always, without a branch -- a branch inside the
                // k-step loop makes the 768-thread kernel spill registers)
                const bool scaled = C::SLDS || __builtin_amdgcn_ballot_w64(odd) != 0;
                const int sc = scaled && tm != 0 ? 13 - ((int)(tm >> 7) - 127) : 0;
                // one 32-channel k-step at a time: its B fragments, then its MFMAs
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    if (C::HALF && ks == C::KS - 1) {
                        // channels 32 ks + 4 g .. +3 on the K = 16 MFMA
                        float x[4];
                        uint32_t w2[2];
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            w2[i] = relu_bf16x2(qc[r][ks][i]);
                            x[2 * i] = bf_lo(w2[i]);
                            x[2 * i + 1] = bf_hi(w2[i]);
                        }
                        const float4 za = *(const float4*)(zh + 32 * ks + 4 * g);
                        den = fmaf(x[0], za.x, den); den = fmaf(x[1], za.y, den);
                        den = fmaf(x[2], za.z, den); den = fmaf(x[3], za.w, den);
                        if (scaled) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[e] = ldexpf(x[e], sc);
                        }
                        if (ROPE) rope4_rotate<2>(x, tab, r4[ks], rope4_rows(r4[ks], ps));
                        typedef __attribute__((ext_vector_type(4))) _Float16 f16x4v;
                        const f16x4v Bq4 = __builtin_bit_cast(
                            f16x4v, u32x2v{pack_f16(x[0], x[1]), pack_f16(x[2], x[3])});
#pragma unroll
                        for (int T = 0; T < C::NT; ++T) {
                            const f16x4v A4 = *(const f16x4v*)(sth + st_off<C::DP>(16 * T + n, 4 * ks + (g >> 1)) +
                                                               4 * (g & 1));
                            acc[T] = __builtin_amdgcn_mfma_f32_16x16x16f16(A4, Bq4, acc[T], 0, 0, 0);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        continue;
                    }
                    const bool live = C::DP == D || 32 * ks + 8 * g < D;
                    u32x4 w4;
                    float x[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        w4[i] = live ? relu_bf16x2(qc[r][ks][i]) : 0u;
                        x[2 * i] = bf_lo(w4[i]);
                        x[2 * i + 1] = bf_hi(w4[i]);
                    }
                    if (C::SLDS) {
                        const float4 za = *(const float4*)(zh + 32 * ks + 8 * g);
                        const float4 zb = *(const float4*)(zh + 32 * ks + 8 * g + 4);
                        den = fmaf(x[0], za.x, den); den = fmaf(x[1], za.y, den);
                        den = fmaf(x[2], za.z, den); den = fmaf(x[3], za.w, den);
                        den = fmaf(x[4], zb.x, den); den = fmaf(x[5], zb.y, den);
                        den = fmaf(x[6], zb.z, den); den = fmaf(x[7], zb.w, den);
                    } else {
                        const bf16x8 Bu = __builtin_bit_cast(bf16x8, w4);
                        dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Azh[C::SLDS ? 0 : ks], Bu, dacc, 0, 0, 0);
                        dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Azl[C::SLDS ? 0 : ks], Bu, dacc, 0, 0, 0);
                    }
                    if (scaled) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[e] = ldexpf(x[e], sc);
                    }
                    if (ROPE) rope4_rotate(x, tab, r4[ks], rope4_rows(r4[ks], ps));
                    u32x4 hw;
#pragma unroll
                    for (int i = 0; i < 4; ++i) hw[i] = pack_f16(x[2 * i], x[2 * i + 1]);
                    const f16x8 Bq = __builtin_bit_cast(f16x8, hw);
#pragma unroll
                    for (int T = 0; T < C::NT; ++T) {
                        const f16x8 A = C::SLDS ? *(const f16x8*)(sth + st_off<C::DP>(16 * T + n, 4 * ks + g))
                                                : A16[C::SLDS ? 0 : T][ks];
                        acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bq, acc[T], 0, 0, 0);
                    }
                    // keep each k-step's LDS reads next to its MFMAs (hoisting
                    // all of them would need 128 more registers a lane)
                    if (C::SLDS) __builtin_amdgcn_sched_barrier(0);
                }
                if (C::SLDS) {
                    den += __shfl_xor(den, 16);
                    den += __shfl_xor(den, 32);
                } else {
                    den = dacc[0];
                }
                den += a.eps;
                // undo the scalings (S by 2^-eS, the group's tokens by 2^sc)
                // and divide; a zero row stays zero, a live row takes the IEEE
                // quotient (NaN or inf only where its denominator is 0 or NaN)
                const float inv = tm != 0 ? ldexpf(1.0f / den, eS - sc) : 0.0f;
#pragma unroll
                for (int sp = 0; sp < C::NT / 2; ++sp) {
                    u32x4 o;
                    o[0] = pack_bf16(acc[2 * sp][0] * inv, acc[2 * sp][1] * inv);
                    o[1] = pack_bf16(acc[2 * sp][2] * inv, acc[2 * sp][3] * inv);
                    o[2] = pack_bf16(acc[2 * sp + 1][0] * inv, acc[2 * sp + 1][1] * inv);
                    o[3] = pack_bf16(acc[2 * sp + 1][2] * inv, acc[2 * sp + 1][3] * inv);
                    if (C::STW)  // (channels past d land in the row's padding chunks)
                        *(u32x4*)(wo + stw_off<C::DP>(n, 4 * sp + g)) = o;
                    else if (C::STG)
                        *(u32x4*)(wo + stg_off(16 * r + n, 4 * sp + g)) = o;
                    else if (C::DP == D || 32 * sp + 8 * g < D)  // part-lines: let L2 merge them
                        buf_store16(o, Or, (uint32_t)(tl * D + 32 * sp + 8 * g) * 2u);
                }
            }
            if (C::STW) {  // the unit out of LDS, 1 KB per streaming store instruction
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int i = 0; i < C::NIW; ++i)
                    buf_store16_stream(*(const u32x4*)(wo + woff[i]), Or,
                                       wok[i] ? (uint32_t)u0 * (2u * D) + (uint32_t)(1024 * i + 16 * lane) : chunk_bytes);
            }
            if (C::STG) {  // whole rows out of LDS, one streaming store per 8 rows
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int i = 0; i < C::NI; ++i) {
                    const int row = C::RPI * i + (lane >> 3);
                    buf_store16_stream(*(const u32x4*)(wo + stg_off(row, lane & 7)), Or,
                                (uint32_t)((u0 + row) * D + 8 * (lane & 7)) * 2u);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32: plain fp32 FMA with S, z in LDS; exact division.
// ---------------------------------------------------------------------------
template <int D>
struct ApplyF32Cfg {
    static constexpr int TT = 32;
    static constexpr int SMEM_FIXED = (D * D + D + 2 * TT * D + 2 * TT) * 4;
};

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void la_apply_f32_kernel(ApplyArgs a) {
    using C = ApplyF32Cfg<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    float* Ss = (float*)smem;        // [D][D]
    float* zs = Ss + D * D;          // [D]
    float* qp = zs + D;              // [TT][D] relu(Q)
    float* qq = qp + C::TT * D;      // [TT][D] RoPE(relu(Q))
    float* dn = qq + C::TT * D;      // [TT] denominators
    int* lv = (int*)(dn + C::TT);    // [TT] 1: relu(Q) of the row is not all zero
    float2* tab = (float2*)(smem + C::SMEM_FIXED);

    const int tid = threadIdx.x;
    int bh, p;
    apply_item_of_block(a.P, a.g.BH, 0, bh, p);
    const int ntok = a.g.ntok;
    const int c0 = p * a.chunk;
    const int c1 = min(c0 + a.chunk, ntok);
    const size_t head = (size_t)bh * ntok * D;
    const float* Qh = (const float*)a.Q + head;
    float* Oh = (float*)a.O + head;

    for (int i = tid; i < D * D; i += 256) Ss[i] = a.S[(size_t)bh * D * D + i];
    if (tid < D) zs[tid] = a.z[(size_t)bh * D + tid];
    int t_lo = 0, nt = 1;
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
    }
    for (int t0 = c0; t0 < c1; t0 += C::TT) {
        lds_barrier();
        for (int i = tid; i < C::TT * D / 2; i += 256) {
            const int tl = i / (D / 2), pp = i % (D / 2);
            const int tok = t0 + tl;
            float x0 = 0.f, x1 = 0.f;
            if (tok < c1) {
                float2 qv = *(const float2*)(Qh + (size_t)tok * D + 2 * pp);
                x0 = fmaxf(qv.x, 0.f);
                x1 = fmaxf(qv.y, 0.f);
            }
            qp[tl * D + 2 * pp] = x0;
            qp[tl * D + 2 * pp + 1] = x1;
            if (ROPE && tok < c1) {
                Pos3 ps = token_pos((uint32_t)(a.g.n_offset + tok), t_lo, a.g);
                rotate(x0, x1, tab[pair_entry(pair_ref(pp, nt, a.g), ps)]);
            }
            qq[tl * D + 2 * pp] = x0;
            qq[tl * D + 2 * pp + 1] = x1;
        }
        lds_barrier();
        if (tid < C::TT) {
            float s = 0.0f;
            bool live = false;
            for (int c = 0; c < D; ++c) {
                s = fmaf(qp[tid * D + c], zs[c], s);
                live = live || qp[tid * D + c] > 0.0f;
            }
            dn[tid] = s + a.eps;
            lv[tid] = live;
        }
        lds_barrier();
        for (int i = tid; i < C::TT * D; i += 256) {
            const int tl = i / D, co = i % D;
            const int tok = t0 + tl;
            if (tok >= c1) continue;
            float s = 0.0f;
            for (int ci = 0; ci < D; ++ci) s = fmaf(qq[tl * D + ci], Ss[ci * D + co], s);
            // a zero row stays zero; a live row takes the IEEE quotient
            Oh[(size_t)tok * D + co] = lv[tl] ? s / dn[tl] : 0.0f;
        }
    }
}
