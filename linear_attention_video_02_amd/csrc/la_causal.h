// Token-causal ReLU linear attention (Eq. 3 of the SANA-Video analysis page,
// section 3.3.1 "Derivation from causal linear attention", with the RoPE of
// section 3.4 at global positions):
//
//   O_i = RoPE(relu Q_i) S_i / (relu(Q_i) . z_i + eps),
//   S_i = S_carry + sum_{j <= i} RoPE(relu K_j)^T V_j,   z_i = z_carry + sum_{j <= i} relu K_j.
//
// Three launches: the state kernel writes one partial (S_p, z_p) per chunk of
// the sequence; la_prefix_kernel turns them, in place, into exclusive
// prefixes (state before the chunk, carry included); la_causal_bf16_kernel
// (la_causal_f32_kernel for fp32 inputs) then scans each chunk with the
// running state on chip.  Without a carry, the bf16 scan at 64 channels on
// chip sums its chunk's prefix from the partials itself (raw_prefix), in the
// prefix kernel's order, and the prefix launch is skipped.
#pragma once

#include "la_common.h"
#include "la_state.h"

// In-place exclusive prefix over the P partials of each head, in the order
// p = 0..P-1, starting from the carry (zeros if none).  Grid (ceil(E/256), B*H),
// one float of (S, z) per thread.  With S_out/z_out, also writes the total
// (the state after the last token).
struct PrefixArgs {
    float* partial;        // [BH][P][D*D + D], partials in, prefixes out
    const float* S_carry;  // [BH][D*D] or null
    const float* z_carry;  // [BH][D] or null
    float* S_out;          // [BH][D*D] or null (may equal S_carry)
    float* z_out;
    int P;
};

template <int D>
__global__ __launch_bounds__(256) void la_prefix_kernel(PrefixArgs a) {
    constexpr int E = D * D + D;
    const int f = blockIdx.x * 256 + threadIdx.x;
    if (f >= E) return;
    const int bh = blockIdx.y;
    float* part = a.partial + (size_t)bh * a.P * E + f;
    float s = 0.0f;
    if (f < D * D) {
        if (a.S_carry) s = a.S_carry[(size_t)bh * D * D + f];
    } else if (a.z_carry) {
        s = a.z_carry[(size_t)bh * D + f - D * D];
    }
    // eight partials at a time: all loads issued before any store (the
    // compiler cannot tell that a store does not alias the next loads)
    for (int p0 = 0; p0 < a.P; p0 += 8) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = p0 + i < a.P ? part[(size_t)(p0 + i) * E] : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (p0 + i < a.P) part[(size_t)(p0 + i) * E] = s;
            s = s + t[i];
        }
    }
    if (f < D * D) {
        if (a.S_out) a.S_out[(size_t)bh * D * D + f] = s;
    } else if (a.z_out) {
        a.z_out[(size_t)bh * D + f - D * D] = s;
    }
}

struct CausalArgs {
    const void* Q;
    const void* K;
    const void* V;
    void* O;
    const float* pre;  // [BH][P][D*D + D]: state before each chunk
    // raw_prefix (bf16, 64 channels on chip): `pre` holds the chunks' own
    // partial states, and the scan of chunk p forms its prefix itself as the
    // prefix kernel would without a carry: 0 + partial 0 + ... + partial p-1
    int raw_prefix = 0;
    float eps;
    int chunk;         // tokens per workgroup (a multiple of 64)
    int P;             // chunks per (batch, head)
    LaGeom g;
};

// ---------------------------------------------------------------------------
// bf16.  Workgroup = 4 waves over one chunk of one head; a step is 64 tokens,
// wave w owns query rows 16w .. 16w+15 of the step.  Channels are padded on
// chip to DP = 64 (d = 32, 64) or 128 (d = 112, 128) with zeros.
//
// Per step:
//  A  the workgroup stages the step's K and V into LDS (16-byte pieces, 8
//     channels of one token per thread and pass):
//     K hi / lo (RoPE(relu K) split in bf16), K u (relu K, exact in bf16) and
//     V' (V with its channels permuted, see below); z partials.
//  B  wave w, for its 16 queries (C = rows: output channels, columns: tokens):
//     inter   acc  = S'^T RoPE(relu Q)^T with S' = running state before the
//             step (bf16 hi + lo in LDS), v_mfma_f32_16x16x32_bf16;
//     intra   for each 16-key block jb <= w:
//             P^T = RoPE(relu K_jb) RoPE(relu Q_w)^T (16 x 16, masked j <= i),
//             acc += V'_jb^T P^T  (v_mfma_f32_16x16x16_bf16, P as hi + lo);
//     den     relu(Q).z (running z) + row sums of the masked relu K relu Q^T;
//     O = acc / (den + eps), one 16-byte store per lane per tile pair.
//  C  the running state S' (fp32 MFMA accumulators held for the whole chunk,
//     32 x 32 tiles: one per wave at DP = 64, a row of four at DP = 128) gets
//     RoPE(relu K)^T V' of the step; its bf16 hi / lo go to LDS for the next
//     step; z likewise.  DP = 64 keeps two LDS copies of the state (step s
//     reads one, writes the other); DP = 128 has room for one, so the waves
//     meet at a barrier after step s's reads before it is overwritten.
//
// V' channel order: value channel co = 32a + 8b + 4c + e is stored at
// p = 32a + 16c + 4b + e.  With it, output tile T row m is value channel
// 32(T/2) + 8(m/4) + 4(T%2) + m%4, so a lane's accumulators of tiles 2s and
// 2s+1 are 8 consecutive channels (one store), and every MFMA operand that
// walks value channels reads 16 consecutive LDS columns.
// ---------------------------------------------------------------------------
template <int D>
struct CausalBf16Cfg {
    static_assert(D == 32 || D == 64 || D == 112 || D == 128, "token-causal kernel: d in {32, 64, 112, 128}");
    static constexpr int DP = D <= 64 ? 64 : 128;   // channels on chip (zero above D)
    static constexpr bool WIDE = DP == 128;
    static constexpr int THREADS = 256;
    static constexpr int NW = 4;
    static constexpr int MINB = WIDE ? 1 : 2;       // workgroups per CU (LDS)
    static constexpr int STEP = 64;                 // tokens per step
    static constexpr int KS = DP / 32;              // 32-channel k-steps
    static constexpr int NT = DP / 16;              // 16-channel output tiles
    static constexpr int TPR = DP / 8;              // staging threads per token row
    static constexpr int SROWS = THREADS / TPR;     // token rows per staging pass
    static constexpr int NJ = STEP / SROWS;         // staging passes per step
    static constexpr int NCB = DP / 32;             // 32-channel blocks
    static constexpr int TPW = NCB * NCB / NW;      // 32 x 32 state tiles per wave
    static constexpr int TILE = STEP * DP;          // bf16 elements of one staged tile
    static constexpr int OFF_KH = 0, OFF_KL = TILE, OFF_KU = 2 * TILE, OFF_V = 3 * TILE;
    static constexpr int OFF_S = 4 * TILE;          // [SBUF buffers][hi, lo][DP x DP] bf16
    static constexpr int STILE = DP * DP;
    static constexpr int SBUF = WIDE ? 1 : 2;
    static constexpr int BYTES_BF16 = (4 * TILE + SBUF * 2 * STILE) * 2;
    static constexpr int OFF_Z = BYTES_BF16;                     // [2][DP] fp32
    static constexpr int OFF_ZP = OFF_Z + 2 * DP * 4;            // [THREADS][8] fp32
    static constexpr int SMEM_FIXED = OFF_ZP + THREADS * 8 * 4;
    static_assert(NJ * SROWS == STEP && TPW * NW == NCB * NCB, "shape");
};

// Element offset of (row, col) in a [rows][DP] bf16 LDS tile: 16-byte chunk c
// of row r is stored at chunk c ^ (r & 7).  Measured on gfx950 at DP = 64
// (cycles per wave instruction, four waves on one CU): 16-byte reads of one
// chunk in 16 consecutive rows 7.3 (8.3 with the chunk permuted by row bits
// 1..3 instead), the state update's transposed 8-byte reads 5.1 (7.8); the
// other accesses here cost the same under both.
template <int DP>
__device__ __forceinline__ int cz(int row, int col) {
    return row * DP + ((((col >> 3) ^ (row & 7))) << 3) + (col & 7);
}

// value channel of permuted position p (inverse of the V' order)
__device__ __forceinline__ int perm_inv(int p) {
    return (p & ~31) + (((p >> 2) & 3) << 3) + (((p >> 4) & 1) << 2) + (p & 3);
}

typedef __attribute__((ext_vector_type(4))) short s16x4v;

template <int D, bool ROPE>
__global__ __launch_bounds__(CausalBf16Cfg<D>::THREADS, CausalBf16Cfg<D>::MINB) void la_causal_bf16_kernel(
    CausalArgs a) {
    using C = CausalBf16Cfg<D>;
    constexpr int DP = C::DP;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* lds = (uint16_t*)smem;
    float* zbuf = (float*)(smem + C::OFF_Z);
    float* zpart = (float*)(smem + C::OFF_ZP);
    float2* tab = (float2*)(smem + C::SMEM_FIXED);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    int bh, p;
    item_of_block(a.P, a.g.BH, bh, p);
    const int ntok = a.g.ntok;
    const int c0 = p * a.chunk;
    const int c1 = min(c0 + a.chunk, ntok);
    const int len = c1 > c0 ? c1 - c0 : 0;
    const int nsteps = (len + C::STEP - 1) / C::STEP;
    const size_t chunk_off = ((size_t)bh * ntok + c0) * D;
    const uint32_t chunk_bytes = (uint32_t)len * D * 2;
    const BufRsrc Qr = make_rsrc((const uint16_t*)a.Q + chunk_off, chunk_bytes);
    const BufRsrc Kr = make_rsrc((const uint16_t*)a.K + chunk_off, chunk_bytes);
    const BufRsrc Vr = make_rsrc((const uint16_t*)a.V + chunk_off, chunk_bytes);
    const BufRsrc Or = make_rsrc((uint16_t*)a.O + chunk_off, chunk_bytes);

    // staging map: thread -> tokens sr + SROWS j of a step, channels 8*sc .. 8*sc+7
    // (channels at or above d: the piece is loaded from channel 0 and zeroed)
    const int sr = tid / C::TPR, sc = tid % C::TPR;
    const bool s_live = DP == D || 8 * sc < D;
    const int s_ch = s_live ? 8 * sc : 0;

    // register ring: step s in slot s & 1
    u32x4 rk[2][C::NJ], rv[2][C::NJ], rq[2][C::KS];
    auto load_kv = [&](int slot, int s) {
        const int t0 = s * C::STEP;
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
            const uint32_t off = (uint32_t)((t0 + sr + C::SROWS * j) * D + s_ch) * 2u;
            rk[slot][j] = buf_load16(Kr, off);
            rv[slot][j] = buf_load16(Vr, off);
        }
    };
    auto q_live = [&](int ks) { return DP == D || 32 * ks + 8 * g < D; };
    auto load_q = [&](int slot, int s) {
        const int t0 = s * C::STEP;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            rq[slot][ks] = buf_load16(
                Qr, (uint32_t)((t0 + 16 * wave + n) * D + (q_live(ks) ? 32 * ks + 8 * g : 0)) * 2u);
    };
    // ---- running state: wave w owns TPW 32 x 32 tiles (ci, cj(t)) of S' ----
    // (fetched before the ring's first loads: loads return in order, and the
    // state is needed first)
    const int m32 = lane & 31, h32 = lane >> 5;
    const int ci = wave * C::TPW / C::NCB;
    auto cj_of = [&](int t) { return (wave * C::TPW + t) % C::NCB; };
    const float* pre = a.pre + ((size_t)bh * a.P + p) * (D * D + D);
    f32x16 sacc[C::TPW];
    float zpre = 0.0f;
    if (C::WIDE || !a.raw_prefix) {
#pragma unroll
        for (int t = 0; t < C::TPW; ++t) {
            const int vc = perm_inv(32 * cj_of(t) + m32);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int k = 32 * ci + 8 * (r >> 2) + 4 * h32 + (r & 3);
                sacc[t][r] = (DP == D || (k < D && vc < D)) ? pre[k * D + vc] : 0.0f;
            }
        }
        zpre = tid < D ? pre[D * D + tid] : 0.0f;
    } else {
        // the prefix from the partials of chunks 0 .. p-1 of this head, NB at
        // a time with all their loads in flight, added in chunk order from 0
        constexpr int NB = 4;
        const float* part0 = a.pre + (size_t)bh * a.P * (D * D + D);
#pragma unroll
        for (int t = 0; t < C::TPW; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[t][r] = 0.0f;
        for (int q0 = 0; q0 < p; q0 += NB) {
            float tv[NB][C::TPW][16], tz[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const float* src = part0 + (size_t)(q0 + u < p ? q0 + u : q0) * (D * D + D);
#pragma unroll
                for (int t = 0; t < C::TPW; ++t) {
                    const int vc = perm_inv(32 * cj_of(t) + m32);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int k = 32 * ci + 8 * (r >> 2) + 4 * h32 + (r & 3);
                        tv[u][t][r] = (DP == D || (k < D && vc < D)) ? src[k * D + vc] : 0.0f;
                    }
                }
                tz[u] = tid < D ? src[D * D + tid] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < NB; ++u)
                if (q0 + u < p) {
#pragma unroll
                    for (int t = 0; t < C::TPW; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) sacc[t][r] = sacc[t][r] + tv[u][t][r];
                    zpre = zpre + tz[u];
                }
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the ring's
    load_kv(0, 0);
    load_q(0, 0);
    load_kv(1, 1);
    load_q(1, 1);

    int t_lo = 0, nt = 1;
    Rope4 rk4{}, rq4[C::KS];
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
        // pairs past d / 2 hold zeros: any table entry rotates them to zeros
        rk4 = rope4_make(s_live ? 4 * sc : 0, nt, a.g);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) rq4[ks] = rope4_make(q_live(ks) ? 16 * ks + 4 * g : 0, nt, a.g);
    }

    // bf16 hi / lo of the tiles, transposed (row = permuted value channel), into S buffer `buf`
    auto write_state = [&](int buf) {
        uint16_t* sh = lds + C::OFF_S + buf * 2 * C::STILE;
        uint16_t* sl = sh + C::STILE;
#pragma unroll
        for (int t = 0; t < C::TPW; ++t) {
            const int prow = 32 * cj_of(t) + m32;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int k0 = 32 * ci + 8 * qd + 4 * h32;
                uint32_t h0, l0, h1, l1;
                split_bf16x2(sacc[t][4 * qd + 0], sacc[t][4 * qd + 1], h0, l0);
                split_bf16x2(sacc[t][4 * qd + 2], sacc[t][4 * qd + 3], h1, l1);
                typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
                *(u32x2*)(sh + cz<DP>(prow, k0)) = u32x2{h0, h1};
                *(u32x2*)(sl + cz<DP>(prow, k0)) = u32x2{l0, l1};
            }
        }
    };
    write_state(0);
    if (tid < DP) zbuf[tid] = zpre;
    lds_barrier();

    uint16_t* kh = lds + C::OFF_KH;
    uint16_t* kl = lds + C::OFF_KL;
    uint16_t* ku = lds + C::OFF_KU;
    uint16_t* vp = lds + C::OFF_V;

    // Two steps per trip, so that each ring slot and state buffer is a fixed
    // set of registers / a fixed LDS offset: with a run-time slot the
    // compiler moves the ring registers at the end of every step and waits
    // for the loads issued in that same step first.  An odd step count runs
    // one more step past the chunk instead of leaving the trip early (an
    // early exit makes the compiler wait for loads one step too soon): its
    // loads read zeros, which add nothing to the state, and its stores are
    // dropped by the bounded descriptor.
    for (int s2 = 0; s2 < nsteps; s2 += 2)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int s = s2 + u;
        const int slot = u, cur = u;
        const int sbuf = C::SBUF == 2 ? cur : 0;  // state buffer read in this step
        const int t0 = s * C::STEP;

        // ---------------- A: stage K and V of this step ----------------
        float zp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) zp[e] = 0.0f;
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
            const int row = sr + C::SROWS * j;
            const u32x4 kraw = s_live ? rk[slot][j] : u32x4{0u, 0u, 0u, 0u};
            const u32x4 vraw = s_live ? rv[slot][j] : u32x4{0u, 0u, 0u, 0u};
            u32x4 ku4;
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = relu_bf16x2(kraw[i]);
                ku4[i] = w;
                x[2 * i] = bf_lo(w);
                x[2 * i + 1] = bf_hi(w);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) zp[e] += x[e];
            if (ROPE) {
                const int tok = min(c0 + t0 + row, c1 - 1);
                rope4_rotate(x, tab, rk4, rope4_rows(rk4, token_pos8((uint32_t)(a.g.n_offset + tok), t_lo, a.g)));
            }
            u32x4 hw, lw;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hh, ll;
                split_bf16x2(x[2 * i], x[2 * i + 1], hh, ll);
                hw[i] = hh;
                lw[i] = ll;
            }
            const int o = cz<DP>(row, 8 * sc);
            *(u32x4*)(kh + o) = hw;
            *(u32x4*)(kl + o) = lw;
            *(u32x4*)(ku + o) = ku4;
            // V': channels 8sc..8sc+3 -> p0 .. p0+3, 8sc+4..+7 -> p0+16 ..
            const int p0 = 32 * (sc >> 2) + 4 * (sc & 3);
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
            *(u32x2*)(vp + cz<DP>(row, p0)) = u32x2{vraw[0], vraw[1]};
            *(u32x2*)(vp + cz<DP>(row, p0 + 16)) = u32x2{vraw[2], vraw[3]};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) zpart[tid * 8 + e] = zp[e];
        // refill the ring with step s + 2: K and V now, Q once this step's
        // queries have been read (below), so that the loads land in the
        // slot's own registers
        load_kv(slot, s + 2);
        lds_barrier();

        // ---------------- B: outputs of this wave's 16 queries ----------------
        const float* zc = zbuf + cur * DP;
        float den = 0.0f;
        uint32_t qbits = 0;  // non-zero iff this lane's relu(Q) values are not all zero
        bf16x8 Bq[C::KS], Bl[C::KS], Bu[C::KS];
        Pos3 qps;
        if (ROPE) qps = token_pos8((uint32_t)(a.g.n_offset + min(c0 + t0 + 16 * wave + n, c1 - 1)), t_lo, a.g);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const u32x4 qraw = q_live(ks) ? rq[slot][ks] : u32x4{0u, 0u, 0u, 0u};
            float x[8];
            u32x4 u4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = relu_bf16x2(qraw[i]);
                u4[i] = w;
                x[2 * i] = bf_lo(w);
                x[2 * i + 1] = bf_hi(w);
            }
            Bu[ks] = __builtin_bit_cast(bf16x8, u4);
            qbits |= (u4[0] | u4[1]) | (u4[2] | u4[3]);
            const float4 za = *(const float4*)(zc + 32 * ks + 8 * g);
            const float4 zb = *(const float4*)(zc + 32 * ks + 8 * g + 4);
            den = fmaf(x[0], za.x, den); den = fmaf(x[1], za.y, den);
            den = fmaf(x[2], za.z, den); den = fmaf(x[3], za.w, den);
            den = fmaf(x[4], zb.x, den); den = fmaf(x[5], zb.y, den);
            den = fmaf(x[6], zb.z, den); den = fmaf(x[7], zb.w, den);
            if (ROPE) {
                rope4_rotate(x, tab, rq4[ks], rope4_rows(rq4[ks], qps));
            }
            u32x4 hw, lw;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hh, ll;
                split_bf16x2(x[2 * i], x[2 * i + 1], hh, ll);
                hw[i] = hh;
                lw[i] = ll;
            }
            Bq[ks] = __builtin_bit_cast(bf16x8, hw);
            Bl[ks] = __builtin_bit_cast(bf16x8, lw);
        }
        load_q(slot, s + 2);

        f32x4 acc[C::NT];
#pragma unroll
        for (int T = 0; T < C::NT; ++T) acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
        // inter: S'^T (running state before the step) times the queries
        {
            const uint16_t* sh = lds + C::OFF_S + sbuf * 2 * C::STILE;
            const uint16_t* sl = sh + C::STILE;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
                for (int T = 0; T < C::NT; ++T) {
                    const int o = cz<DP>(16 * T + n, 32 * ks + 8 * g);
                    const bf16x8 Ah = *(const bf16x8*)(sh + o);
                    const bf16x8 Al = *(const bf16x8*)(sl + o);
                    acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bq[ks], acc[T], 0, 0, 0);
                    acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, Bq[ks], acc[T], 0, 0, 0);
                    acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bl[ks], acc[T], 0, 0, 0);
                }
        }
        // intra: key blocks 0 .. wave of this step
        for (int jb = 0; jb <= wave; ++jb) {
            f32x4 c1v = f32x4{0.f, 0.f, 0.f, 0.f}, cuv = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int o = cz<DP>(16 * jb + n, 32 * ks + 8 * g);
                const bf16x8 Ah = *(const bf16x8*)(kh + o);
                const bf16x8 Al = *(const bf16x8*)(kl + o);
                const bf16x8 Au = *(const bf16x8*)(ku + o);
                c1v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bq[ks], c1v, 0, 0, 0);
                c1v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, Bq[ks], c1v, 0, 0, 0);
                c1v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bl[ks], c1v, 0, 0, 0);
                cuv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Au, Bu[ks], cuv, 0, 0, 0);
            }
            // lane (n, g) holds keys j = 16jb + 4g + r for query i = 16*wave + n
            if (jb == wave) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r > n) {
                        c1v[r] = 0.0f;
                        cuv[r] = 0.0f;
                    }
            }
            den += (cuv[0] + cuv[1]) + (cuv[2] + cuv[3]);
            uint32_t ph0, pl0, ph1, pl1;
            split_bf16x2(c1v[0], c1v[1], ph0, pl0);
            split_bf16x2(c1v[2], c1v[3], ph1, pl1);
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
            const s16x4v Ph = __builtin_bit_cast(s16x4v, u32x2{ph0, ph1});
            const s16x4v Pl = __builtin_bit_cast(s16x4v, u32x2{pl0, pl1});
#pragma unroll
            for (int T = 0; T < C::NT; ++T) {
                // V'^T tile: lane m gets tokens 16jb+4g .. +3 of permuted channel 16T + m
                const s16x4v Av = lds_read_tr4(vp + cz<DP>(16 * jb + 4 * g + (n >> 2), 16 * T + 4 * (n & 3)));
                acc[T] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Av, Ph, acc[T], 0, 0, 0);
                acc[T] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Av, Pl, acc[T], 0, 0, 0);
            }
        }
        den += __shfl_xor(den, 16);
        den += __shfl_xor(den, 32);
        den += a.eps;
        // a zero row stays zero; a live row takes the IEEE quotient (NaN or
        // inf only where its denominator is 0 or NaN)
        qbits |= (uint32_t)__shfl_xor((int)qbits, 16);
        qbits |= (uint32_t)__shfl_xor((int)qbits, 32);
        const float inv = qbits != 0 ? 1.0f / den : 0.0f;
        {
            const int tl = t0 + 16 * wave + n;
#pragma unroll
            for (int sp = 0; sp < C::NT / 2; ++sp) {
                u32x4 o;
                o[0] = pack_bf16(acc[2 * sp][0] * inv, acc[2 * sp][1] * inv);
                o[1] = pack_bf16(acc[2 * sp][2] * inv, acc[2 * sp][3] * inv);
                o[2] = pack_bf16(acc[2 * sp + 1][0] * inv, acc[2 * sp + 1][1] * inv);
                o[3] = pack_bf16(acc[2 * sp + 1][2] * inv, acc[2 * sp + 1][3] * inv);
                if (DP == D || 32 * sp + 8 * g < D)  // value channels 32sp + 8g .. +7
                    buf_store16_stream(o, Or, (uint32_t)(tl * D + 32 * sp + 8 * g) * 2u);
            }
        }

        // ---------------- C: add this step to the running state ----------------
        {
            const int rd_row = 8 * h32 + ((lane & 15) >> 2);
            const int rd_col = 4 * (lane & 3);
            const int kc = 32 * ci + 16 * ((lane >> 4) & 1) + rd_col;  // key channel column of the tr read
#pragma unroll
            for (int k16 = 0; k16 < C::STEP / 16; ++k16) {
                const int r0 = 16 * k16 + rd_row;
                const bf16x8 Ah = lds_read_tr8(kh + cz<DP>(r0, kc), kh + cz<DP>(r0 + 4, kc));
                const bf16x8 Al = lds_read_tr8(kl + cz<DP>(r0, kc), kl + cz<DP>(r0 + 4, kc));
#pragma unroll
                for (int t = 0; t < C::TPW; ++t) {
                    const int vc = 32 * cj_of(t) + 16 * ((lane >> 4) & 1) + rd_col;  // permuted value column
                    const bf16x8 Bv = lds_read_tr8(vp + cz<DP>(r0, vc), vp + cz<DP>(r0 + 4, vc));
                    sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, Bv, sacc[t], 0, 0, 0);
                    sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Al, Bv, sacc[t], 0, 0, 0);
                }
            }
            if (C::SBUF == 1) lds_barrier();  // every wave's reads of the one state copy done
            write_state(C::SBUF == 2 ? cur ^ 1 : 0);
            if (tid < DP) {
                // z partials of the SROWS threads holding channel tid, in thread order
                float sum = 0.0f;
                for (int r = 0; r < C::SROWS; ++r) sum += zpart[(r * C::TPR + (tid >> 3)) * 8 + (tid & 7)];
                zbuf[(cur ^ 1) * DP + tid] = zc[tid] + sum;
            }
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs: plain fp32 arithmetic (no matrix cores), the running state in
// LDS.  Workgroup = 256 threads over one chunk of one head, steps of 16
// tokens:
//  1. stage relu(K) (z and denominator), RoPE(relu K), V, relu(Q),
//     RoPE(relu Q) of the step;
//  2. thread (i, j) forms the two masked step scores RoPE(relu Q_i).RoPE(relu K_j)
//     and relu(Q_i).relu(K_j) (j <= i); the denominator of row i is
//     relu(Q_i).z + its row of unrotated scores + eps;
//  3. thread (channel c, row group) forms O_i[c] = (sum_k RoPE(relu Q_i)[k] S[k][c]
//     + sum_{j <= i} score_ij V_j[c]) / den_i;
//  4. S[k][c] += sum_j RoPE(relu K_j)[k] V_j[c], z += sum_j relu(K_j).
// Sums run in a fixed order, so results repeat bitwise.
// ---------------------------------------------------------------------------
template <int D>
struct CausalF32Cfg {
    static constexpr int THREADS = 256;
    static constexpr int T = 16;                       // tokens per step
    static constexpr int G = THREADS / D;              // row groups of the output phase
    static constexpr int RG = T / G;                   // rows per group
    static constexpr int NE = (D * D + THREADS - 1) / THREADS;  // state entries per thread
    static constexpr int OFF_S = 0;                    // [D][D] running state
    static constexpr int OFF_Z = OFF_S + D * D * 4;    // [D]
    static constexpr int OFF_KU = OFF_Z + D * 4;       // [T][D] relu K
    static constexpr int OFF_KR = OFF_KU + T * D * 4;  // [T][D] RoPE(relu K)
    static constexpr int OFF_V = OFF_KR + T * D * 4;   // [T][D] V
    static constexpr int OFF_QU = OFF_V + T * D * 4;   // [T][D] relu Q
    static constexpr int OFF_QR = OFF_QU + T * D * 4;  // [T][D] RoPE(relu Q)
    static constexpr int OFF_A = OFF_QR + T * D * 4;   // [T][T] rotated scores (masked)
    static constexpr int OFF_AU = OFF_A + T * T * 4;   // [T][T] unrotated scores (masked)
    static constexpr int OFF_DEN = OFF_AU + T * T * 4; // [T] 1 / den, 0 for a zero row
    static constexpr int SMEM_FIXED = OFF_DEN + T * 4;
    static_assert(G >= 1 && T % G == 0, "row groups");
};

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void la_causal_f32_kernel(CausalArgs a) {
    using C = CausalF32Cfg<D>;
    constexpr int T = C::T;
    extern __shared__ __align__(16) unsigned char smem[];
    float* S = (float*)(smem + C::OFF_S);
    float* zs = (float*)(smem + C::OFF_Z);
    float* ku = (float*)(smem + C::OFF_KU);
    float* kr = (float*)(smem + C::OFF_KR);
    float* vv = (float*)(smem + C::OFF_V);
    float* qu = (float*)(smem + C::OFF_QU);
    float* qr = (float*)(smem + C::OFF_QR);
    float* A = (float*)(smem + C::OFF_A);
    float* Au = (float*)(smem + C::OFF_AU);
    float* rden = (float*)(smem + C::OFF_DEN);
    float2* tab = (float2*)(smem + C::SMEM_FIXED);

    const int tid = threadIdx.x;
    int bh, p;
    item_of_block(a.P, a.g.BH, bh, p);
    const int ntok = a.g.ntok;
    const int c0 = p * a.chunk;
    const int c1 = min(c0 + a.chunk, ntok);
    const size_t head = (size_t)bh * ntok * D;
    const float* Qh = (const float*)a.Q + head;
    const float* Kh = (const float*)a.K + head;
    const float* Vh = (const float*)a.V + head;
    float* Oh = (float*)a.O + head;

    int t_lo = 0, nt = 1;
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
    }
    // the state before the chunk (exclusive prefix, carry included)
    const float* pre = a.pre + ((size_t)bh * a.P + p) * (D * D + D);
    for (int e = tid; e < D * D; e += C::THREADS) S[e] = pre[e];
    if (tid < D) zs[tid] = pre[D * D + tid];

    // output phase: channel oc, rows og*RG .. og*RG + RG - 1 (threads past G*D idle)
    const int oc = tid % D, og = tid / D;
    for (int t0 = c0; t0 < c1; t0 += T) {
        lds_barrier();  // the previous step's reads done (and the prefix visible)
        // ---- 1. stage the step (rows past the chunk are zeros) ----
        for (int i = tid; i < T * D / 2; i += C::THREADS) {
            const int tl = i / (D / 2), pp = i % (D / 2);
            const int tok = t0 + tl;
            float2 k2 = {0.f, 0.f}, v2 = {0.f, 0.f}, q2 = {0.f, 0.f};
            if (tok < c1) {
                k2 = *(const float2*)(Kh + (size_t)tok * D + 2 * pp);
                v2 = *(const float2*)(Vh + (size_t)tok * D + 2 * pp);
                q2 = *(const float2*)(Qh + (size_t)tok * D + 2 * pp);
            }
            float k0 = fmaxf(k2.x, 0.f), k1 = fmaxf(k2.y, 0.f);
            float q0 = fmaxf(q2.x, 0.f), q1 = fmaxf(q2.y, 0.f);
            const int o = tl * D + 2 * pp;
            ku[o] = k0;
            ku[o + 1] = k1;
            qu[o] = q0;
            qu[o + 1] = q1;
            vv[o] = v2.x;
            vv[o + 1] = v2.y;
            if (ROPE && tok < c1) {
                const Pos3 ps = token_pos((uint32_t)(a.g.n_offset + tok), t_lo, a.g);
                const float2 cs = tab[pair_entry(pair_ref(pp, nt, a.g), ps)];
                rotate(k0, k1, cs);
                rotate(q0, q1, cs);
            }
            kr[o] = k0;
            kr[o + 1] = k1;
            qr[o] = q0;
            qr[o + 1] = q1;
        }
        lds_barrier();
        // ---- 2. masked step scores, thread (i, j) ----
        {
            const int i = tid / T, j = tid % T;
            float sr = 0.f, su = 0.f;
            if (j <= i) {
                for (int k = 0; k < D; ++k) {
                    sr = fmaf(qr[i * D + k], kr[j * D + k], sr);
                    su = fmaf(qu[i * D + k], ku[j * D + k], su);
                }
            }
            A[i * T + j] = sr;
            Au[i * T + j] = su;
        }
        lds_barrier();
        if (tid < T) {
            const int i = tid;
            float den = 0.f, any = 0.f;
            for (int k = 0; k < D; ++k) {
                den = fmaf(qu[i * D + k], zs[k], den);
                any = fmaxf(any, qu[i * D + k]);
            }
            for (int j = 0; j <= i; ++j) den += Au[i * T + j];
            den += a.eps;
            // a zero row stays zero; a live row takes the IEEE quotient
            rden[i] = any > 0.f ? 1.0f / den : 0.0f;
        }
        lds_barrier();
        // ---- 3. outputs ----
        if (og < C::G) {
            float num[C::RG];
#pragma unroll
            for (int r = 0; r < C::RG; ++r) num[r] = 0.f;
            for (int k = 0; k < D; ++k) {
                const float s = S[k * D + oc];
#pragma unroll
                for (int r = 0; r < C::RG; ++r) num[r] = fmaf(qr[(og * C::RG + r) * D + k], s, num[r]);
            }
#pragma unroll
            for (int r = 0; r < C::RG; ++r) {
                const int i = og * C::RG + r;
                float intra = 0.f;
                for (int j = 0; j <= i; ++j) intra = fmaf(A[i * T + j], vv[j * D + oc], intra);
                const int tok = t0 + i;
                if (tok < c1) Oh[(size_t)tok * D + oc] = (num[r] + intra) * rden[i];
            }
        }
        lds_barrier();  // every read of S before the update
        // ---- 4. state update ----
#pragma unroll
        for (int m = 0; m < C::NE; ++m) {
            const int e = tid + C::THREADS * m;
            if (e < D * D) {
                const int k = e / D, c = e % D;
                float s = S[e];
                float add = 0.f;
#pragma unroll
                for (int j = 0; j < T; ++j) add = fmaf(kr[j * D + k], vv[j * D + c], add);
                S[e] = s + add;
            }
        }
        if (tid < D) {
            float add = 0.f;
#pragma unroll
            for (int j = 0; j < T; ++j) add += ku[j * D + tid];
            zs[tid] += add;
        }
    }
}
