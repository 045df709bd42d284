// State pass of ReLU linear attention (the two sums of the linear-attention
// equation on the SANA-Video analysis page, section 3.4, in the Eq. 2 form):
//
//   S = sum_j RoPE(relu(K_j))^T V_j   (d x d, fp32)      z = sum_j relu(K_j)   (d, fp32)
//
// Work split: P workgroups per (batch, head).  Workgroup p of head bh reduces
// the token chunk [p*chunk, (p+1)*chunk) to a partial (S_p, z_p) in the
// workspace.  Stage 2 sums the P partials of each head in the fixed order
// p = 0..P-1, adds the carried state when there is one (block-causal mode,
// Eq. 3 / Algorithm 1) and writes S and z.  Results are bitwise reproducible
// for a given shape.  Stage 2 runs in one of two ways, with identical sums:
//  - bf16 kernel, fused: the partials are written with device-scope stores
//    and the last workgroup of a head to finish (a per-head counter in the
//    workspace, tagged with the call's epoch and put back to zero by the
//    workgroup that completes the head) does the sum.  No release
//    fence: a device-scope fence per workgroup would write back a whole XCD
//    L2 each time.  Used while a head's partials are at most 256 KB (the
//    tuning knob state_fused = 1 forces it).
//  - separate launch (la_state_combine_kernel): the kernel boundary makes
//    the partials visible, and the sum is spread over many workgroups.
//    Used by the fp32 kernel, by the token-causal pass (its prefix kernel
//    reads the partials), for larger partials and with state_fused = 0.
#pragma once

#include "la_common.h"

struct CombineArgs {
    const float* partial;  // [BH][P][D*D + D]
    float* S_out;          // [BH][D*D]
    float* z_out;          // [BH][D]
    float* S_out2;         // optional second destination (block commit)
    float* z_out2;
    const float* S_carry;  // optional addend (block mode)
    const float* z_carry;
    int P;
    int BH;
};

struct StateArgs {
    const void* K;
    const void* V;
    float* partial;        // [BH][pslots][D*D + D]
    int chunk;             // tokens per workgroup
    int P;                 // workgroups per (batch, head): chunks 0 .. P-1
    int pslots;            // partial slots per (batch, head), >= P
    LaGeom g;
    // Stage 2 inside the bf16 kernel (ticket != null): the last workgroup of
    // a head to finish sums that head's partials (see the kernel's end).
    // Counters hold (epoch << 32) | count: a call counts from zero in its own
    // epoch, so a count left by a call that never completed is raised past.
    // The workgroup that completes a head puts its counter back to zero, so
    // a captured launch replayed with its one epoch starts from zero too.
    unsigned long long* ticket;  // [BH]
    unsigned epoch;              // this call's epoch (never 0)
    CombineArgs cmb;
};

// Stage 2: grid (ceil(E4 / 256), B*H), one float4 of (S, z) per thread.  Sums
// the P partials in the fixed order p = 0..P-1 (sixteen partials' loads in
// flight before they are added: one round trip for P <= 16), then adds the
// carry: S_b = carry + sum_p S_p.
template <int D>
__global__ __launch_bounds__(256) void la_state_combine_kernel(CombineArgs a) {
    constexpr int E = D * D + D;
    constexpr int E4 = E / 4;  // S and z regions both hold whole float4s (D % 4 == 0)
    const int f = blockIdx.x * 256 + threadIdx.x;
    const int bh = blockIdx.y;
    if (f >= E4) return;
    const float4* part = (const float4*)(a.partial + (size_t)bh * a.P * E);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int NB = 16;
    for (int p = 0; p < a.P; p += NB) {
        float4 v[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u)
            if (p + u < a.P) v[u] = part[(size_t)(p + u) * E4 + f];
#pragma unroll
        for (int u = 0; u < NB; ++u)
            if (p + u < a.P) {
                s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
            }
    }
    const int e = 4 * f;
    if (e < D * D) {
        const size_t o = (size_t)bh * D * D + e;
        if (a.S_carry) {
            const float4 c = *(const float4*)(a.S_carry + o);
            s.x = c.x + s.x; s.y = c.y + s.y; s.z = c.z + s.z; s.w = c.w + s.w;
        }
        *(float4*)(a.S_out + o) = s;
        if (a.S_out2) *(float4*)(a.S_out2 + o) = s;
    } else {
        const size_t o = (size_t)bh * D + (e - D * D);
        if (a.z_carry) {
            const float4 c = *(const float4*)(a.z_carry + o);
            s.x = c.x + s.x; s.y = c.y + s.y; s.z = c.z + s.z; s.w = c.w + s.w;
        }
        *(float4*)(a.z_out + o) = s;
        if (a.z_out2) *(float4*)(a.z_out2 + o) = s;
    }
}

// ---------------------------------------------------------------------------
// Work item of a workgroup: (head, chunk).  Workgroups are dealt round-robin
// to the 8 XCDs by linear id; this mapping gives XCD x a contiguous run of
// items (whole heads) instead of one chunk position of every head.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void item_of_block(int P, int BH, int& bh, int& p) {
    const int T = P * BH;
    const int i = blockIdx.x;
    const int k = (T % 8 == 0) ? (i % 8) * (T / 8) + i / 8 : i;
    bh = k / P;
    p = k % P;
}

// ---------------------------------------------------------------------------
// bf16 inputs: MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation.
//
// One workgroup per CU (two workgroups sharing a CU run at unequal speed:
// the sequencer favours older waves).  d <= 64: 1024 threads (4 waves per
// SIMD, <= 128 registers a lane); d = 128: 512 threads.
//
// Per tile of TT tokens: every thread loads 16-byte pieces (8 channels of one
// token) of K and V through bounded buffer descriptors, coalesced.  K gets
// relu, the z partial (un-rotated), RoPE at the token's global grid position,
// and a split into bf16 hi + lo (hi + lo = RoPE(relu K) to 2^-16: a single
// bf16 rounding costs up to ~2% in rows whose sum over tokens cancels, e.g.
// the pair partners of outlier channels).  hi, lo and V go to LDS row-major
// (row = token, no padding) with one 16-byte write each; 32-channel column
// blocks are XOR-swizzled by row so that the four rows a transposed read
// touches fall in distinct banks.  MFMA operands -- 8 consecutive tokens of
// one channel -- come back with two ds_read_b64_tr_b16.
// MFMA: C[c_in][c_out] += A[c_in][tok] B[tok][c_out], A = (hi, lo)^T, B = V.
// Wave w owns key-channel tile w % NCI (32 rows of S), value-channel split
// (w / NCI) % NVS (all value channels, or at d = 64 one 32-channel half) and
// token group w / (NCI NVS) of every tile; at the end the NTG token groups of
// each key-channel tile are summed in LDS in a fixed order (a tree of fan-in four).
// Two LDS buffers: tile t's MFMAs read one while tile t+1 is staged into the
// other, with one barrier per tile.  DEPTH tiles of K/V are in flight per
// workgroup (a register ring refilled right after each tile is staged).
// ---------------------------------------------------------------------------
template <int D, int THR = (D <= 64 ? 1024 : 512)>
struct StateBf16Cfg {
    static constexpr int DP = Pad<D>::P;      // channels on chip (zero above D)
    static constexpr int THREADS = THR;
    static constexpr int NW = THREADS / 64;
    static constexpr int CH = DP / 8;         // 16-byte pieces per token row
    static constexpr int ROWS = THREADS / CH; // token rows per load pass
    static constexpr int LP = D <= 64 ? 1 : 2;  // load passes per tile
    static constexpr int TT = ROWS * LP;      // tokens per tile: 256, 128, 64 (half at 512 threads, d <= 64)
    static constexpr int DEPTH = 2;           // tiles of K/V in flight per workgroup
    static constexpr int TILE = TT * DP;      // elements per LDS tile
    static constexpr int BUF = 3 * TILE;      // K hi, K lo, V
    static constexpr int NCI = DP / 32;       // key-channel tiles
    // Value channels split over the waves at d = 64: each wave then owns one
    // 32 x 32 tile of S, and the fold at the end moves half the bytes through
    // LDS in one level instead of two (it took 1.44 us of the 720p-5s pass).
    // The extra K fragment reads per tile cost nothing visible.  At d >= 112
    // the staging VALU bounds the loop and the split is not used.
    static constexpr int NVS = D == 64 ? 2 : 1;
    static constexpr int NCO = NCI * NVS;     // (key tile, value split) pairs
    static constexpr int NTG = NW / NCO;      // token groups
    static constexpr int NJ = DP / 32 / NVS;  // value-channel tiles per wave
    static constexpr int KSTEPS = TT / (16 * NTG);  // 16-token steps per wave per tile
    static constexpr int NACC = NJ * 16;      // accumulators per lane
    static constexpr int STAGE_BYTES = 2 * BUF * 2;
    // fold of the token groups in groups of four: the first level has the
    // most senders, NTG - ceil(NTG / 4) per (key tile, value split) pair
    static constexpr int RED_BYTES = (NTG - (NTG + 3) / 4) * NCO * 64 * NACC * 4;
    static constexpr int ZRED_BYTES = NW * DP * 4;  // z: one row of DP sums per wave
    static constexpr int m1 = STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES;
    static constexpr int SMEM_FIXED = m1 > ZRED_BYTES ? m1 : ZRED_BYTES;
    static_assert(KSTEPS >= 1 && KSTEPS * 16 * NTG == TT, "k-steps");
    static_assert((NTG & (NTG - 1)) == 0, "token groups: power of two");
};

// Element offset of (row, ch) in a swizzled row-major tile: 32-channel block
// b of row r is stored at block b ^ s(r), with s chosen per d so that rows
// r0..r0+3 (r0 % 4 == 0) start in different 16-bank groups.
template <int D>
__device__ __forceinline__ int swz(int row, int ch) {
    const int s = D == 32 ? 0 : (D == 64 ? ((row >> 1) & 1) : (row & 3));  // D = on-chip width
    return row * D + (((ch >> 5) ^ s) << 5) + (ch & 31);
}

// One level of the z reduce-scatter (partner lane ^ MSK) and the levels
// after it: a lane holding NV channel sums keeps half (the upper half if its
// MSK bit is set) and adds the partner's copy of that half; once one value
// is left, the remaining levels add plainly.  coff tracks the first channel
// held.  Every channel's sum is formed pair for pair as the full butterfly
// forms it.
template <int NV, int MSK>
__device__ __forceinline__ void z_scatter(float (&zp)[8], int lane, int& coff) {
    if constexpr (MSK < 64) {
        if constexpr (NV > 1) {
            constexpr int H = NV / 2;
            const bool hi = (lane & MSK) != 0;
#pragma unroll
            for (int e = 0; e < H; ++e) {
                const float keep = hi ? zp[H + e] : zp[e];
                const float send = hi ? zp[e] : zp[H + e];
                zp[e] = keep + __shfl_xor(send, MSK);
            }
            coff += hi ? H : 0;
            z_scatter<H, MSK * 2>(zp, lane, coff);
        } else {
            zp[0] += __shfl_xor(zp[0], MSK);
            z_scatter<1, MSK * 2>(zp, lane, coff);
        }
    }
}

template <int D, bool ROPE, int THR = StateBf16Cfg<D>::THREADS>
__global__ __launch_bounds__(THR) void la_state_bf16_kernel(StateArgs a) {
    using C = StateBf16Cfg<D, THR>;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* lds = (uint16_t*)smem;   // [2][3][TT*D]: buffer, (K hi, K lo, V)
    float2* tab = (float2*)(smem + C::SMEM_FIXED);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: branches on it stay scalar)
    int bh, p;
    item_of_block(a.P, a.g.BH, bh, p);
    const int ntok = a.g.ntok;
    const int c0 = p * a.chunk;
    const int c1 = min(c0 + a.chunk, ntok);
    // K and V of this chunk through descriptors bounded to [c0, c1): tokens
    // past c1 read as zeros, which add nothing to S or z.
    const size_t chunk_off = ((size_t)bh * ntok + c0) * D;
    const uint32_t chunk_bytes = c1 > c0 ? (uint32_t)(c1 - c0) * D * 2 : 0u;
    const BufRsrc Kr = make_rsrc((const uint16_t*)a.K + chunk_off, chunk_bytes);
    const BufRsrc Vr = make_rsrc((const uint16_t*)a.V + chunk_off, chunk_bytes);
    const int cc = tid % C::CH, trow = tid / C::CH;
    // lanes past the real channels (d = 112 only) load out of range: zeros
    const bool live = C::DP == D || 8 * cc < D;

    // ring of DEPTH tiles in registers: tile i lives in slot i % DEPTH
    u32x4 kr[C::DEPTH][C::LP], vr[C::DEPTH][C::LP];
    auto load_tile = [&](u32x4 (&kk)[C::LP], u32x4 (&vv)[C::LP], int tile) {
#pragma unroll
        for (int j = 0; j < C::LP; ++j) {
            const uint32_t off = live ? (uint32_t)((tile * C::TT + trow + j * C::ROWS) * D + 8 * cc) * 2u : chunk_bytes;
            kk[j] = buf_load16(Kr, off);
            vv[j] = buf_load16(Vr, off);
        }
    };
#pragma unroll
    for (int s = 0; s < C::DEPTH; ++s) load_tile(kr[s], vr[s], s);

    int t_lo = 0;
    Rope4 r4{};
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        int nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
        r4 = rope4_make(live ? 4 * cc : 0, nt, a.g);
    }

    float zp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zp[e] = 0.0f;

    // stage tile `tile` (held in ring slot s) into LDS buffer `buf`
    auto stage = [&](int s, int buf, int tile) {
        uint16_t* khi = lds + buf * C::BUF;
        uint16_t* klo = khi + C::TILE;
        uint16_t* vt = klo + C::TILE;
#pragma unroll
        for (int j = 0; j < C::LP; ++j) {
            const int tl = trow + j * C::ROWS;
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = relu_bf16x2(kr[s][j][i]);
                x[2 * i] = bf_lo(w);
                x[2 * i + 1] = bf_hi(w);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) zp[e] += x[e];
            if (ROPE) {
                const int tok = min(c0 + tile * C::TT + tl, c1 - 1);
                rope4_rotate(x, tab, r4, rope4_rows(r4, token_pos8((uint32_t)(a.g.n_offset + tok), t_lo, a.g)));
            }
            u32x4 hw, lw;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t h, l;
                split_bf16x2(x[2 * i], x[2 * i + 1], h, l);
                hw[i] = h;
                lw[i] = l;
            }
            const int o = swz<C::DP>(tl, 8 * cc);
            *(u32x4*)(khi + o) = hw;
            *(u32x4*)(klo + o) = lw;
            *(u32x4*)(vt + o) = vr[s][j];
        }
    };

    f32x16 acc[C::NJ];
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

    // transposed-read addressing: 16-lane group (q, g) reads rows
    // kb0 + 8g + 4h + i16/4, columns 32*tile + 16q + 4*(i16%4)
    const int i16 = lane & 15, q = (lane >> 4) & 1, gq = lane >> 5, m = lane & 31;
    const int rd_row = 8 * gq + (i16 >> 2);
    const int rd_col = 16 * q + 4 * (i16 & 3);
    const int ctile = wave % C::NCI;   // key-channel tile of this wave
    const int vsp = (wave / C::NCI) % C::NVS;  // value-channel split of this wave
    const int co = ctile * C::NVS + vsp;       // its (key tile, value split) pair
    const int tgrp = wave / C::NCO;    // token group of this wave

    const int ntiles = c1 > c0 ? (c1 - c0 + C::TT - 1) / C::TT : 0;
    // The loop sits inside this branch so that it is entered only after tile
    // 0 is staged and tile DEPTH requested: reachable straight from the ring's
    // first loads, the loop made the compiler wait for every load in flight
    // at every other tile.
    if (ntiles > 0) {
        lds_barrier();  // RoPE table complete
        stage(0, 0, 0);
        load_tile(kr[0], vr[0], C::DEPTH);
        lds_barrier();
    // Whole rounds of the ring, no early exit: tiles past the chunk end are
    // zeros from the bounded descriptor and add nothing, and a uniform trip
    // count keeps the compiler's count of outstanding loads exact.
    for (int tb = 0; tb < ntiles; tb += C::DEPTH) {
#pragma unroll
        for (int s = 0; s < C::DEPTH; ++s) {
            const int t = tb + s;            // tile consumed now, in LDS buffer s & 1
            const int cur = s & 1;           // (DEPTH is even)
            const uint16_t* khi = lds + cur * C::BUF;
            const uint16_t* klo = khi + C::TILE;
            const uint16_t* vt = klo + C::TILE;
            bf16x8 Ah[C::KSTEPS], Al[C::KSTEPS], Bv[C::KSTEPS][C::NJ];
#pragma unroll
            for (int st = 0; st < C::KSTEPS; ++st) {
                const int kb0 = 16 * (tgrp * C::KSTEPS + st);
                const int r0 = kb0 + rd_row, r1 = r0 + 4;
                const int col = 32 * ctile + rd_col;
                Ah[st] = lds_read_tr8(khi + swz<C::DP>(r0, col), khi + swz<C::DP>(r1, col));
                Al[st] = lds_read_tr8(klo + swz<C::DP>(r0, col), klo + swz<C::DP>(r1, col));
#pragma unroll
                for (int j = 0; j < C::NJ; ++j) {
                    const int vcol = 32 * (vsp * C::NJ + j) + rd_col;
                    Bv[st][j] = lds_read_tr8(vt + swz<C::DP>(r0, vcol), vt + swz<C::DP>(r1, vcol));
                }
            }
            // stage the next tile into the other buffer while these MFMAs run
            const int sn = (s + 1) % C::DEPTH;
            stage(sn, cur ^ 1, t + 1);
            load_tile(kr[sn], vr[sn], t + 1 + C::DEPTH);
#pragma unroll
            for (int st = 0; st < C::KSTEPS; ++st)
#pragma unroll
                for (int j = 0; j < C::NJ; ++j) {
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah[st], Bv[st][j], acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Al[st], Bv[st][j], acc[j], 0, 0, 0);
                }
            lds_barrier();
        }
    }
    }

    // ---- fold the token groups of each key-channel tile: a tree of fan-in
    //      four in a fixed order, level by level (group g += g + l, then
    //      g + 2l, then g + 3l, for l = 1, 4, 16, ...) ----
    f32x4* red = (f32x4*)smem;
    static_assert(C::RED_BYTES <= C::SMEM_FIXED, "reduction buffer");
    static_assert(C::NACC % 4 == 0, "fold in 16-byte pieces");
    lds_barrier();
#pragma unroll
    for (int lvl = 1; lvl < C::NTG; lvl *= 4) {
        const int k = (tgrp % (4 * lvl)) / lvl;  // position in the group of four
        const bool member = tgrp % lvl == 0;
        const int base = (tgrp / (4 * lvl)) * 3;  // first slot of this group
        if (member && k > 0) {
            const int slot = (base + k - 1) * C::NCO + co;
#pragma unroll
            for (int j = 0; j < C::NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; r += 4)
                    red[(slot * (C::NACC / 4) + j * 4 + r / 4) * 64 + lane] =
                        f32x4{acc[j][r], acc[j][r + 1], acc[j][r + 2], acc[j][r + 3]};
        }
        lds_barrier();
        if (member && k == 0) {
#pragma unroll
            for (int m = 1; m < 4; ++m) {
                if (tgrp + m * lvl >= C::NTG) break;
                const int slot = (base + m - 1) * C::NCO + co;
#pragma unroll
                for (int j = 0; j < C::NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; r += 4) {
                        const f32x4 v = red[(slot * (C::NACC / 4) + j * 4 + r / 4) * 64 + lane];
                        acc[j][r] += v[0];
                        acc[j][r + 1] += v[1];
                        acc[j][r + 2] += v[2];
                        acc[j][r + 3] += v[3];
                    }
            }
        }
        lds_barrier();
    }

    // ---- write this workgroup's partial (token group 0 holds the sums) ----
    // In the fused mode the partials are device-coherent stores (sc1: written
    // through to the agent-wide coherence point, not left in this XCD's L2).
    // With one partial per head (fused, P = 1) it is the head's sum: S and z
    // are written directly, formed as stage 2 forms them (0 + the partial,
    // then the carry), and the counters are not touched.
    const bool fused = a.ticket != nullptr;
    const bool direct = fused && a.P == 1;
    const CombineArgs& cd = a.cmb;
    auto put = [&](float* dst, float v) {
        if (fused)
            __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            *dst = v;
    };
    constexpr int E = D * D + D;
    float* part = a.partial + ((size_t)bh * a.pslots + p) * E;
    // The sums go to LDS as rows (stride SR floats), and every thread then
    // writes 16 contiguous bytes of the partial at a time (from the MFMA
    // layout directly, a lane would store single words, up to 64 a lane).
    constexpr int SR = C::DP + 4;
    static_assert(C::DP * SR * 4 <= C::SMEM_FIXED, "partial staging");
    float* srow = (float*)smem;
    if (tgrp == 0) {
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * ctile + 8 * (r >> 2) + 4 * gq + (r & 3);
                srow[row * SR + 32 * (vsp * C::NJ + j) + m] = acc[j][r];
            }
    }
    lds_barrier();
    {
        const BufRsrc pr16 = make_rsrc(part, (uint32_t)D * D * 4u);
        for (int f = tid; f < D * D / 4; f += C::THREADS) {
            const int row = f / (D / 4), c4 = f % (D / 4);
            const f32x4 v4 = *(const f32x4*)(srow + row * SR + 4 * c4);
            if (direct) {
                const size_t o = (size_t)bh * D * D + 4 * f;  // row-major S: element 4f
                f32x4 sum = f32x4{0.0f, 0.0f, 0.0f, 0.0f} + v4;
                if (cd.S_carry) sum = *(const f32x4*)(cd.S_carry + o) + sum;
                *(f32x4*)(cd.S_out + o) = sum;
                if (cd.S_out2) *(f32x4*)(cd.S_out2 + o) = sum;
                continue;
            }
            const u32x4 v = __builtin_bit_cast(u32x4, v4);
            if (fused)
                buf_store16_dev(v, pr16, (uint32_t)f * 16u);
            else
                buf_store16(v, pr16, (uint32_t)f * 16u);
        }
    }
    lds_barrier();  // the rows are read before the z sums reuse the LDS
    // ---- z partial: the lanes of a wave that share a channel block (lane
    //      % CH) summed across lanes, then the waves' sums in wave order.
    //      Across lanes as a reduce-scatter: at each level of the butterfly
    //      (partner lane ^ msk) a lane keeps half of its channels and adds the
    //      partner's copy of that half, so each level moves half as many
    //      values as the one before: 7 cross-lane moves a lane at d = 64
    //      instead of 24, whose LDS-crossbar permutes took 1.2 us at the end of
    //      the 720p-5s pass.  The additions are those of the full butterfly,
    //      pair for pair, so z is unchanged bitwise. ----
    float* zr = (float*)smem;  // [NW][DP]
    if constexpr (C::CH <= 8) {
        int coff = 0;  // first channel (within the lane's block of 8) still held
        z_scatter<8, C::CH>(zp, lane, coff);
        // lanes past the last halving hold copies: the first 64 / 2^(levels
        // after it) lanes write, one channel each
        constexpr int WR = C::CH == 4 ? 32 : 64;
        if (lane < WR) zr[wave * C::DP + 8 * (lane % C::CH) + coff] = zp[0];
    } else {
        // 128 channels on chip: two levels only, as a full butterfly (the
        // reduce-scatter's selects do not fit the 512-thread kernel's
        // registers there)
#pragma unroll
        for (int msk = C::CH; msk < 64; msk <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) zp[e] += __shfl_xor(zp[e], msk);
        if (lane < C::CH) {
#pragma unroll
            for (int e = 0; e < 8; ++e) zr[wave * C::DP + 8 * lane + e] = zp[e];
        }
    }
    lds_barrier();
    if (tid < D) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) sum += zr[w * C::DP + tid];
        if (direct) {
            const size_t o = (size_t)bh * D + tid;
            float zs = 0.0f + sum;
            if (cd.z_carry) zs = cd.z_carry[o] + zs;
            cd.z_out[o] = zs;
            if (cd.z_out2) cd.z_out2[o] = zs;
        } else {
            put(&part[D * D + tid], sum);
        }
    }
    if (!fused || direct) return;

    // ---- fused stage 2.  Every thread waits until its partial stores have
    // completed (sc1 stores complete at the device coherence point), then one
    // device-scope atomic per workgroup counts the finished partials of the
    // head.  The workgroup that brings the count to P reads all P partials
    // with device-coherent loads (sc1) and sums them in the fixed order
    // p = 0..P-1 -- the same sums as the separate combine kernel.  No L2
    // write-back or invalidate is needed: the partials never live in L2. ----
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt unconstrained
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    lds_barrier();  // every thread's stores done; zr reads done (flag reuses zr[0])
    int* flag = (int*)smem;
    if (tid == 0) {
        // the head's counter moves to this call's epoch (count 0) unless a
        // workgroup of this call got there first; then count this partial
        __hip_atomic_fetch_max(&a.ticket[bh], (unsigned long long)a.epoch << 32, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long old =
            __hip_atomic_fetch_add(&a.ticket[bh], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = (unsigned)old == (unsigned)(a.P - 1);
    }
    lds_barrier();
    if (*flag) {
        // every workgroup of the head has counted: no other update can follow
        if (tid == 0) __hip_atomic_store(&a.ticket[bh], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const CombineArgs& c = a.cmb;
        constexpr int E4 = E / 4;  // S and z regions both hold whole float4s
        const BufRsrc hp = make_rsrc(c.partial + (size_t)bh * c.P * E, (uint32_t)c.P * E * 4u);
        for (int f = tid; f < E4; f += C::THREADS) {
            f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int q0 = 0; q0 < c.P; q0 += 8) {
                u32x4 v[8];  // eight partials' loads in flight, then added in order
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = buf_load16_dev(hp, (uint32_t)((q0 + u) * E4 + f) * 16u);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (q0 + u < c.P) s += __builtin_bit_cast(f32x4, v[u]);
            }
            const int e = 4 * f;
            if (e < D * D) {
                const size_t o = (size_t)bh * D * D + e;
                if (c.S_carry) s = *(const f32x4*)(c.S_carry + o) + s;
                *(f32x4*)(c.S_out + o) = s;
                if (c.S_out2) *(f32x4*)(c.S_out2 + o) = s;
            } else {
                const size_t o = (size_t)bh * D + (e - D * D);
                if (c.z_carry) s = *(const f32x4*)(c.z_carry + o) + s;
                *(f32x4*)(c.z_out + o) = s;
                if (c.z_out2) *(f32x4*)(c.z_out2 + o) = s;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs: plain fp32 FMA (full input precision), 32-token LDS tiles.
// Thread t owns the state entries t, t+256, ... (row = e / d, col = e % d).
// ---------------------------------------------------------------------------
template <int D>
struct StateF32Cfg {
    static constexpr int TT = 32;
    static constexpr int NE = D * D / 256;
    static constexpr int SMEM_FIXED = 3 * TT * D * 4;
};

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void la_state_f32_kernel(StateArgs a) {
    using C = StateF32Cfg<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    float* kp = (float*)smem;      // relu(K)
    float* kq = kp + C::TT * D;    // RoPE(relu(K))
    float* vv = kq + C::TT * D;    // V
    float2* tab = (float2*)(smem + C::SMEM_FIXED);
    const int tid = threadIdx.x;
    int bh, p;
    item_of_block(a.P, a.g.BH, bh, p);
    const int ntok = a.g.ntok;
    const int c0 = p * a.chunk;
    const int c1 = min(c0 + a.chunk, ntok);
    const size_t head = (size_t)bh * ntok * D;
    const float* Kh = (const float*)a.K + head;
    const float* Vh = (const float*)a.V + head;

    int t_lo = 0, nt = 1;
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
    }
    float acc[C::NE];
#pragma unroll
    for (int j = 0; j < C::NE; ++j) acc[j] = 0.0f;
    float zacc = 0.0f;

    for (int t0 = c0; t0 < c1; t0 += C::TT) {
        lds_barrier();
        for (int i = tid; i < C::TT * D / 2; i += 256) {
            const int tl = i / (D / 2), pp = i % (D / 2);
            const int tok = t0 + tl;
            float x0 = 0.f, x1 = 0.f, v0 = 0.f, v1 = 0.f;
            if (tok < c1) {
                float2 kk = *(const float2*)(Kh + (size_t)tok * D + 2 * pp);
                float2 vv2 = *(const float2*)(Vh + (size_t)tok * D + 2 * pp);
                x0 = fmaxf(kk.x, 0.f); x1 = fmaxf(kk.y, 0.f); v0 = vv2.x; v1 = vv2.y;
            }
            kp[tl * D + 2 * pp] = x0;
            kp[tl * D + 2 * pp + 1] = x1;
            if (ROPE && tok < c1) {
                Pos3 ps = token_pos((uint32_t)(a.g.n_offset + tok), t_lo, a.g);
                rotate(x0, x1, tab[pair_entry(pair_ref(pp, nt, a.g), ps)]);
            }
            kq[tl * D + 2 * pp] = x0;
            kq[tl * D + 2 * pp + 1] = x1;
            vv[tl * D + 2 * pp] = v0;
            vv[tl * D + 2 * pp + 1] = v1;
        }
        lds_barrier();
        for (int tl = 0; tl < C::TT; ++tl) {
#pragma unroll
            for (int j = 0; j < C::NE; ++j) {
                const int e = tid + 256 * j;
                acc[j] = fmaf(kq[tl * D + e / D], vv[tl * D + e % D], acc[j]);
            }
            if (tid < D) zacc += kp[tl * D + tid];
        }
    }
    constexpr int E = D * D + D;
    float* part = a.partial + ((size_t)bh * a.pslots + p) * E;
#pragma unroll
    for (int j = 0; j < C::NE; ++j) part[tid + 256 * j] = acc[j];
    if (tid < D) part[D * D + tid] = zacc;
}
