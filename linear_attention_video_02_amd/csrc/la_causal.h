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
// then scans each chunk in 64-token steps with the running state on chip.
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
    float eps;
    int chunk;         // tokens per workgroup (a multiple of 64)
    int P;             // chunks per (batch, head)
    LaGeom g;
};

// ---------------------------------------------------------------------------
// bf16, d = 64.  Workgroup = 4 waves over one chunk of one head; a step is 64
// tokens, wave w owns query rows 16w .. 16w+15 of the step.
//
// Per step:
//  A  every thread stages 2 tokens x 8 channels of K and V into LDS:
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
//  C  wave w adds RoPE(relu K)^T V' of the step to its 32 x 32 tile of the
//     running state (fp32 MFMA accumulators held for the whole chunk) and
//     writes the tile's bf16 hi / lo for the next step; z likewise.
//
// V' channel order: value channel co = 32a + 8b + 4c + e is stored at
// p = 32a + 16c + 4b + e.  With it, output tile T row m is value channel
// 32(T/2) + 8(m/4) + 4(T%2) + m%4, so a lane's accumulators of tiles 2s and
// 2s+1 are 8 consecutive channels (one store), and every MFMA operand that
// walks value channels reads 16 consecutive LDS columns.
// ---------------------------------------------------------------------------
template <int D>
struct CausalBf16Cfg {
    static_assert(D == 64, "token-causal kernel: d = 64");
    static constexpr int THREADS = 256;
    static constexpr int NW = 4;
    static constexpr int STEP = 64;                 // tokens per step
    static constexpr int KS = D / 32;               // 32-channel k-steps
    static constexpr int NT = D / 16;               // 16-channel output tiles
    static constexpr int TILE = STEP * D;           // bf16 elements of one staged tile
    static constexpr int OFF_KH = 0, OFF_KL = TILE, OFF_KU = 2 * TILE, OFF_V = 3 * TILE;
    static constexpr int OFF_S = 4 * TILE;          // [2 buffers][hi, lo][D x D] bf16
    static constexpr int STILE = D * D;
    static constexpr int BYTES_BF16 = (4 * TILE + 4 * STILE) * 2;
    static constexpr int OFF_Z = BYTES_BF16;                     // [2][D] fp32
    static constexpr int OFF_ZP = OFF_Z + 2 * D * 4;             // [THREADS][8] fp32
    static constexpr int SMEM_FIXED = OFF_ZP + THREADS * 8 * 4;
};

// Element offset of (row, col) in a [rows][64] bf16 LDS tile: 16-byte chunk c
// of row r is stored at chunk c ^ (r & 7).  Measured on gfx950 (cycles per
// wave instruction, four waves on one CU): 16-byte reads of one chunk in 16
// consecutive rows 7.3 (8.3 with the chunk permuted by row bits 1..3
// instead), the state update's transposed 8-byte reads 5.1 (7.8); the other
// accesses here cost the same under both.
__device__ __forceinline__ int cz(int row, int col) {
    return row * 64 + ((((col >> 3) ^ (row & 7))) << 3) + (col & 7);
}

// value channel of permuted position p (inverse of the V' order)
__device__ __forceinline__ int perm_inv(int p) {
    return (p & ~31) + (((p >> 2) & 3) << 3) + (((p >> 4) & 1) << 2) + (p & 3);
}

typedef __attribute__((ext_vector_type(4))) short s16x4v;

template <int D, bool ROPE>
__global__ __launch_bounds__(CausalBf16Cfg<D>::THREADS, 2) void la_causal_bf16_kernel(CausalArgs a) {
    using C = CausalBf16Cfg<D>;
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

    // staging map: thread -> tokens sr and sr + 32 of a step, channels 8*sc .. 8*sc+7
    const int sr = tid >> 3, sc = tid & 7;

    // register ring: step s in slot s & 1
    u32x4 rk[2][2], rv[2][2], rq[2][C::KS];
    auto load_kv = [&](int slot, int s) {
        const int t0 = s * C::STEP;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t off = (uint32_t)((t0 + sr + 32 * j) * D + 8 * sc) * 2u;
            rk[slot][j] = buf_load16(Kr, off);
            rv[slot][j] = buf_load16(Vr, off);
        }
    };
    auto load_q = [&](int slot, int s) {
        const int t0 = s * C::STEP;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            rq[slot][ks] = buf_load16(Qr, (uint32_t)((t0 + 16 * wave + n) * D + 32 * ks + 8 * g) * 2u);
    };
    // ---- running state: wave w owns the 32 x 32 tile (ci, cj) of S' ----
    // (fetched before the ring's first loads: loads return in order, and the
    // state is needed first)
    const int m32 = lane & 31, h32 = lane >> 5;
    const int ci = wave >> 1, cj = wave & 1;
    const float* pre = a.pre + ((size_t)bh * a.P + p) * (D * D + D);
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int k = 32 * ci + 8 * (r >> 2) + 4 * h32 + (r & 3);
        sacc[r] = pre[k * D + perm_inv(32 * cj + m32)];
    }
    const float zpre = tid < D ? pre[D * D + tid] : 0.0f;
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the ring's
    load_kv(0, 0);
    load_q(0, 0);
    load_kv(1, 1);
    load_q(1, 1);

    int t_lo = 0, nt = 1;
    PairRef prk[4], prq[C::KS][4];
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
#pragma unroll
        for (int i = 0; i < 4; ++i) prk[i] = pair_ref(4 * sc + i, nt, a.g);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) prq[ks][i] = pair_ref(16 * ks + 4 * g + i, nt, a.g);
    }

    // bf16 hi / lo of the tile, transposed (row = permuted value channel), into S buffer `buf`
    auto write_state = [&](int buf) {
        uint16_t* sh = lds + C::OFF_S + buf * 2 * C::STILE;
        uint16_t* sl = sh + C::STILE;
        const int prow = 32 * cj + m32;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int k0 = 32 * ci + 8 * qd + 4 * h32;
            uint32_t h0, l0, h1, l1;
            split_bf16x2(sacc[4 * qd + 0], sacc[4 * qd + 1], h0, l0);
            split_bf16x2(sacc[4 * qd + 2], sacc[4 * qd + 3], h1, l1);
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
            *(u32x2*)(sh + cz(prow, k0)) = u32x2{h0, h1};
            *(u32x2*)(sl + cz(prow, k0)) = u32x2{l0, l1};
        }
    };
    write_state(0);
    if (tid < D) zbuf[tid] = zpre;
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
        const int t0 = s * C::STEP;

        // ---------------- A: stage K and V of this step ----------------
        float zp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) zp[e] = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = sr + 32 * j;
            u32x4 ku4;
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = relu_bf16x2(rk[slot][j][i]);
                ku4[i] = w;
                x[2 * i] = bf_lo(w);
                x[2 * i + 1] = bf_hi(w);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) zp[e] += x[e];
            if (ROPE) {
                const int tok = min(c0 + t0 + row, c1 - 1);
                const Pos3 ps = token_pos((uint32_t)(a.g.n_offset + tok), t_lo, a.g);
#pragma unroll
                for (int i = 0; i < 4; ++i) rotate(x[2 * i], x[2 * i + 1], tab[pair_entry(prk[i], ps)]);
            }
            u32x4 hw, lw;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hh, ll;
                split_bf16x2(x[2 * i], x[2 * i + 1], hh, ll);
                hw[i] = hh;
                lw[i] = ll;
            }
            const int o = cz(row, 8 * sc);
            *(u32x4*)(kh + o) = hw;
            *(u32x4*)(kl + o) = lw;
            *(u32x4*)(ku + o) = ku4;
            // V': channels 8sc..8sc+3 -> p0 .. p0+3, 8sc+4..+7 -> p0+16 ..
            const int p0 = 32 * (sc >> 2) + 4 * (sc & 3);
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
            *(u32x2*)(vp + cz(row, p0)) = u32x2{rv[slot][j][0], rv[slot][j][1]};
            *(u32x2*)(vp + cz(row, p0 + 16)) = u32x2{rv[slot][j][2], rv[slot][j][3]};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) zpart[tid * 8 + e] = zp[e];
        // refill the ring with step s + 2: K and V now, Q once this step's
        // queries have been read (below), so that the loads land in the
        // slot's own registers
        load_kv(slot, s + 2);
        lds_barrier();

        // ---------------- B: outputs of this wave's 16 queries ----------------
        const float* zc = zbuf + cur * D;
        float den = 0.0f;
        bf16x8 Bq[C::KS], Bl[C::KS], Bu[C::KS];
        Pos3 qps;
        if (ROPE) qps = token_pos((uint32_t)(a.g.n_offset + min(c0 + t0 + 16 * wave + n, c1 - 1)), t_lo, a.g);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            float x[8];
            u32x4 u4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = relu_bf16x2(rq[slot][ks][i]);
                u4[i] = w;
                x[2 * i] = bf_lo(w);
                x[2 * i + 1] = bf_hi(w);
            }
            Bu[ks] = __builtin_bit_cast(bf16x8, u4);
            const float4 za = *(const float4*)(zc + 32 * ks + 8 * g);
            const float4 zb = *(const float4*)(zc + 32 * ks + 8 * g + 4);
            den = fmaf(x[0], za.x, den); den = fmaf(x[1], za.y, den);
            den = fmaf(x[2], za.z, den); den = fmaf(x[3], za.w, den);
            den = fmaf(x[4], zb.x, den); den = fmaf(x[5], zb.y, den);
            den = fmaf(x[6], zb.z, den); den = fmaf(x[7], zb.w, den);
            if (ROPE) {
#pragma unroll
                for (int i = 0; i < 4; ++i) rotate(x[2 * i], x[2 * i + 1], tab[pair_entry(prq[ks][i], qps)]);
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
            const uint16_t* sh = lds + C::OFF_S + cur * 2 * C::STILE;
            const uint16_t* sl = sh + C::STILE;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
                for (int T = 0; T < C::NT; ++T) {
                    const int o = cz(16 * T + n, 32 * ks + 8 * g);
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
                const int o = cz(16 * jb + n, 32 * ks + 8 * g);
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
                const s16x4v Av = lds_read_tr4(vp + cz(16 * jb + 4 * g + (n >> 2), 16 * T + 4 * (n & 3)));
                acc[T] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Av, Ph, acc[T], 0, 0, 0);
                acc[T] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Av, Pl, acc[T], 0, 0, 0);
            }
        }
        den += __shfl_xor(den, 16);
        den += __shfl_xor(den, 32);
        den += a.eps;
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
        {
            const int tl = t0 + 16 * wave + n;
#pragma unroll
            for (int sp = 0; sp < C::NT / 2; ++sp) {
                u32x4 o;
                o[0] = pack_bf16(acc[2 * sp][0] * inv, acc[2 * sp][1] * inv);
                o[1] = pack_bf16(acc[2 * sp][2] * inv, acc[2 * sp][3] * inv);
                o[2] = pack_bf16(acc[2 * sp + 1][0] * inv, acc[2 * sp + 1][1] * inv);
                o[3] = pack_bf16(acc[2 * sp + 1][2] * inv, acc[2 * sp + 1][3] * inv);
                buf_store16_stream(o, Or, (uint32_t)(tl * D + 32 * sp + 8 * g) * 2u);
            }
        }

        // ---------------- C: add this step to the running state ----------------
        {
            const int rd_row = 8 * h32 + ((lane & 15) >> 2);
            const int rd_col = 4 * (lane & 3);
            const int kc = 32 * ci + 16 * ((lane >> 4) & 1) + rd_col;  // key channel column of the tr read
            const int vc = 32 * cj + 16 * ((lane >> 4) & 1) + rd_col;  // permuted value column
#pragma unroll
            for (int k16 = 0; k16 < C::STEP / 16; ++k16) {
                const int r0 = 16 * k16 + rd_row;
                const bf16x8 Ah = lds_read_tr8(kh + cz(r0, kc), kh + cz(r0 + 4, kc));
                const bf16x8 Al = lds_read_tr8(kl + cz(r0, kc), kl + cz(r0 + 4, kc));
                const bf16x8 Bv = lds_read_tr8(vp + cz(r0, vc), vp + cz(r0 + 4, vc));
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, Bv, sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Al, Bv, sacc, 0, 0, 0);
            }
            write_state(cur ^ 1);
            if (tid < D) {
                // z partials of the 32 threads holding channel tid, in thread order
                float sum = 0.0f;
                for (int r = 0; r < 32; ++r) sum += zpart[(r * 8 + (tid >> 3)) * 8 + (tid & 7)];
                zbuf[(cur ^ 1) * D + tid] = zc[tid] + sum;
            }
        }
        lds_barrier();
    }
}
