// Apply pass of ReLU linear attention (numerator / denominator of Eq. 2 on the
// SANA-Video analysis page, section 3.4 "Integration of 3D RoPE"):
//
//   O_i = RoPE(relu(Q_i)) S / (relu(Q_i) . z + eps)
//
// One HBM read of Q and one write of O; S and z (a few KB per head) come from
// L2.  Rows with relu(Q_i) = 0 produce exact zeros.
#pragma once

#include "la_common.h"

struct ApplyArgs {
    const void* Q;
    void* O;
    const float* S;  // [BH][D*D]
    const float* z;  // [BH][D]
    float eps;
    int chunk;       // tokens per workgroup
    int P;           // workgroups per (batch, head)
    int ilv;         // bf16: 1 = the head's workgroups take interleaved units of the whole head
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
// One 512-thread workgroup (8 waves; 4 at d = 128) per CU over a chunk of one head; each
// wave takes UNIT-token units of the chunk from an LDS queue and keeps DEPTH
// units of Q in flight.
// ---------------------------------------------------------------------------
template <int D>
struct ApplyBf16Cfg {
    static constexpr int DP = Pad<D>::P;  // channels on chip (zero above D)
    // d <= 64: 8 waves per CU (2 per SIMD: S^T hi + lo in registers);
    // d >= 112: 12 waves (S^T in LDS, <= 168 registers a lane)
    static constexpr int THREADS = D <= 64 ? 512 : 768;
    static constexpr int NW = THREADS / 64;
    static constexpr int KS = DP / 32;  // 32-channel k-steps
    static constexpr int NT = DP / 16;  // 16-channel output tiles
    static constexpr int GR = D <= 64 ? 2 : 1;   // 16-token groups per unit of work
    static constexpr int UNIT = 16 * GR;         // tokens a wave takes from the queue at a time
    static constexpr int DEPTH = D <= 64 ? 3 : 2;  // units of Q in flight per wave
    // d >= 112: S^T (fp16) lives in LDS instead of registers (128 x 128
    // fp16 would take 128 registers a lane); MFMA A fragments are read from it
    static constexpr bool SLDS = DP > 64;
    // d = 64: Q and O pass through a per-wave LDS tile so that every global
    // load / store instruction moves 8 whole 128-byte rows (the MFMA operand
    // layout would touch 16 rows per instruction, half of each line).
    static constexpr bool STG = D == 64;
    static constexpr int RPI = 8;                          // rows per staged load / store
    static constexpr int NI = UNIT / RPI;                  // staged loads per unit (= GR * KS)
    static constexpr int ZBYTES = DP * 4;                  // z, S^T, staging, then the RoPE table
    // d <= 64: S^T in fp32 (row stride d + 4), read once into the fragments
    static constexpr int SROW = D + 4;
    static constexpr int SBYTES = SLDS ? DP * DP * 2 : D * SROW * 4;
    static constexpr int STGBYTES = STG ? NW * 2 * UNIT * D * 2 : 0;
    static constexpr int FIXED = ZBYTES + SBYTES + STGBYTES;
    static_assert(!STG || NI == GR * KS, "staged unit = register ring slot");
};

// Element offset of row r, 16-byte chunk c of a wave's staging tile
// ([UNIT][64] bf16): chunk c of row r sits at c ^ f(r), which keeps both the
// row-major 8-rows-per-instruction accesses and the MFMA-layout accesses
// (16 consecutive rows at one chunk) free of bank conflicts.
__device__ __forceinline__ int stg_off(int r, int c) {
    return r * 64 + ((c ^ ((r ^ (r >> 3)) & 7)) << 3);
}

// Element offset of S^T row pr (= 16 T + m, see below), 16-byte chunk c, in
// the LDS copy used at d >= 112: chunks are XOR-swizzled by row so that 16
// consecutive rows read at one chunk hit 16 distinct bank groups.
template <int DP>
__device__ __forceinline__ int st_off(int pr, int c) {
    return pr * DP + ((c ^ (pr & 15)) << 3);
}

// Work item mapping shared with the state pass (whole heads per XCD).
__device__ __forceinline__ void apply_item_of_block(int P, int BH, int& bh, int& p) {
    const int T = P * BH;
    const int i = blockIdx.x;
    const int k = (T % 8 == 0) ? (i % 8) * (T / 8) + i / 8 : i;
    bh = k / P;
    p = k % P;
}

template <int D, bool ROPE>
__global__ __launch_bounds__(ApplyBf16Cfg<D>::THREADS) void la_apply_bf16_kernel(ApplyArgs a) {
    using C = ApplyBf16Cfg<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    float* zs = (float*)smem;                        // [DP] z (zero above d)
    uint16_t* st = (uint16_t*)(smem + C::ZBYTES);    // [DP][DP] S^T hi (d >= 112)
    uint16_t* stg = (uint16_t*)(smem + C::ZBYTES + C::SBYTES);  // [NW][Q, O][UNIT][D] (d = 64)
    float2* tab = (float2*)(smem + C::FIXED);
    __shared__ int q_next;  // next unit of this workgroup's chunk, in tokens
    __shared__ float smax[C::NW];  // per-wave max |S|

    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g = lane >> 4;
    int bh, p;
    apply_item_of_block(a.P, a.g.BH, bh, p);
    const int ntok = a.g.ntok;
    const bool ilv = a.ilv != 0;
    const int c0 = ilv ? 0 : p * a.chunk;
    const int c1 = ilv ? ntok : min(c0 + a.chunk, ntok);
    const int len = c1 > c0 ? c1 - c0 : 0;
    // queue position q (in tokens) -> first token of the unit, within [c0, c1)
    auto tok_of = [&](int q) -> int { return ilv ? ((q / C::UNIT) * a.P + p) * C::UNIT : q; };
    // Q and O of this chunk through descriptors bounded to [c0, c1): rows
    // past c1 read as zeros and their stores are dropped.
    const size_t chunk_off = ((size_t)bh * ntok + c0) * D;
    const uint32_t chunk_bytes = (uint32_t)len * D * 2;
    const BufRsrc Qr = make_rsrc((const uint16_t*)a.Q + chunk_off, chunk_bytes);
    const BufRsrc Or = make_rsrc((uint16_t*)a.O + chunk_off, chunk_bytes);

    if (threadIdx.x == 0) q_next = C::NW * C::DEPTH * C::UNIT;  // the first units are pre-assigned
    // Units of UNIT tokens are taken from the workgroup's queue, so waves that
    // run faster (the sequencer favours older waves) take more of the chunk.
    auto grab = [&]() -> int {
        int v = 0;
        if (lane == 0) v = atomicAdd(&q_next, C::UNIT);
        return __builtin_amdgcn_readfirstlane(v);
    };
    u32x4 qr[C::DEPTH][C::GR][C::KS];
    auto load_unit = [&](u32x4 (&q)[C::GR][C::KS], int u0) {
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
            for (int ks = 0; ks < C::KS; ++ks)
                q[r][ks] = buf_load16(Qr, (uint32_t)(tl * D + 32 * ks + 8 * g) * 2u);
        }
    };
    // d <= 64: S and this lane's z entries are fetched before the first Q
    // loads.  Loads return in order, so fetched after them the conversion
    // below (and every wave's first MFMA) would wait until all of the first
    // units of Q had arrived -- at kernel start, when every CU asks at once,
    // that is several microseconds.  S comes in with coalesced 16-byte loads
    // (a lane's fragment entries lie in 8 different rows of S, which as
    // single-word global loads would be 64 per lane) and goes to LDS
    // transposed, where each lane reads its fragments as 16-byte rows.
    // (d >= 112 likewise: S comes in with the same coalesced loads, ahead of
    // Q's, and goes from registers straight into the fp16 copy in LDS.)
    const float* Sh = a.S + (size_t)bh * D * D;
    constexpr int S4 = (D * D / 4 + C::THREADS - 1) / C::THREADS;  // float4s a thread
    f32x4 sraw[S4];
    float zraw[C::SLDS ? 1 : C::KS][8];
#pragma unroll
    for (int i = 0; i < S4; ++i) {
        const int f = threadIdx.x + i * C::THREADS;
        if (f < D * D / 4) sraw[i] = *(const f32x4*)(Sh + 4 * f);
    }
    if (!C::SLDS) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) zraw[ks][e] = a.z[(size_t)bh * D + 32 * ks + 8 * g + e];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of Q's
    // first DEPTH units of each wave: fixed, so their loads go out before the
    // prologue work
    const int wave = threadIdx.x >> 6;
    int us[C::DEPTH];
#pragma unroll
    for (int s = 0; s < C::DEPTH; ++s) {
        us[s] = tok_of((s * C::NW + wave) * C::UNIT);
        load_unit(qr[s], us[s]);
    }

    // S^T fragments (fp16, scaled by 2^-eS) and this lane's z entries
    f16x8 A16[C::SLDS ? 1 : C::NT][C::KS];
    float* sT = (float*)st;  // d <= 64: [D][SROW] fp32, sT[co][ci] = S[ci][co]
    float amax = 0.0f;       // this thread's largest |S| entry
#pragma unroll
    for (int i = 0; i < S4; ++i) {
        const int f = threadIdx.x + i * C::THREADS;
        if (f < D * D / 4) {
            const int ci = f / (D / 4), co = 4 * (f % (D / 4));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!C::SLDS) sT[(co + j) * C::SROW + ci] = sraw[i][j];
                amax = fmaxf(amax, fabsf(sraw[i][j]));
            }
        }
    }
    amax = wave_max(amax);
    if (lane == 0) smax[wave] = amax;
    // eS: the head's largest |S| times 2^-eS lies in [2^13, 2^14) (read after
    // a barrier that follows the smax writes)
    auto head_scale = [&]() -> int {
        float hmax = 0.0f;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) hmax = fmaxf(hmax, smax[w]);
        int e = 0;
        if (hmax > 0.0f) {
            (void)frexpf(hmax, &e);
            e -= 14;
        }
        return e;
    };
    int eS = 0;
    if (C::SLDS) {
        lds_barrier();
        eS = head_scale();
        // row pr = 16 T + m of the copy holds value channel co(T, m), the MFMA
        // row order used below; element k is S[k][co] 2^-eS (zero past d)
        auto put_st = [&](int k, int co, float sv) {
            const int T = 2 * (co >> 5) + ((co >> 2) & 1);
            const int m = (((co >> 3) & 3) << 2) | (co & 3);
            st[st_off<C::DP>(16 * T + m, k >> 3) + (k & 7)] =
                __builtin_bit_cast(uint16_t, (_Float16)ldexpf(sv, -eS));
        };
#pragma unroll
        for (int i = 0; i < S4; ++i) {
            const int f = threadIdx.x + i * C::THREADS;
            if (f < D * D / 4) {
                const int k = f / (D / 4), co = 4 * (f % (D / 4));
#pragma unroll
                for (int j = 0; j < 4; ++j) put_st(k, co + j, sraw[i][j]);
            }
        }
        // the padding rows and columns (key or value channel >= d)
        for (int e = threadIdx.x; e < C::DP * C::DP - D * D; e += C::THREADS) {
            int k, co;
            if (e < D * (C::DP - D)) {
                k = e / (C::DP - D);
                co = D + e % (C::DP - D);
            } else {
                k = D + (e - D * (C::DP - D)) / C::DP;
                co = (e - D * (C::DP - D)) % C::DP;
            }
            put_st(k, co, 0.0f);
        }
    }
    if (C::SLDS)  // (d <= 64 sums the denominator on the MFMA from registers)
        for (int c = threadIdx.x; c < C::DP; c += C::THREADS) zs[c] = c < D ? a.z[(size_t)bh * D + c] : 0.0f;
    // d <= 64: the denominator relu(q).z runs on the MFMA too, with z as an A
    // tile of 16 identical rows (bf16 hi + lo) and the un-rotated relu(q) --
    // exact in bf16 -- as B: every accumulator of a token's lanes is its sum.
    bf16x8 Azh[C::SLDS ? 1 : C::KS], Azl[C::SLDS ? 1 : C::KS];
    if (!C::SLDS) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float zv = zraw[ks][e];
                const __bf16 hi = (__bf16)zv;
                Azh[ks][e] = hi;
                Azl[ks][e] = (__bf16)(zv - (float)hi);
            }
    }

    int t_lo = 0, nt = 1;
    PairRef pr[C::KS][4];
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pr[ks][i] = pair_ref((C::DP == D || 32 * ks + 8 * g < D) ? 16 * ks + 4 * g + i : 0, nt, a.g);
    }
    lds_barrier();  // RoPE table, S^T copy, per-wave max |S| and queue head visible
    if (!C::SLDS) eS = head_scale();
    // this lane's S^T fragments: value channel co(T, n), key channels
    // 32 ks + 8 g .. +7 -- two 16-byte LDS reads each
#pragma unroll
    for (int T = 0; T < (C::SLDS ? 0 : C::NT); ++T) {
        const int co = 32 * (T >> 1) + 8 * (n >> 2) + 4 * (T & 1) + (n & 3);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const f32x4 v0 = *(const f32x4*)(sT + co * C::SROW + 32 * ks + 8 * g);
            const f32x4 v1 = *(const f32x4*)(sT + co * C::SROW + 32 * ks + 8 * g + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) A16[T][ks][e] = (_Float16)ldexpf(e < 4 ? v0[e] : v1[e - 4], -eS);
        }
    }

    bool more = true;
    while (more) {
#pragma unroll
        for (int s = 0; s < C::DEPTH; ++s) {
            const int u0 = us[s];
            if (u0 >= len) {  // units are taken in increasing order: nothing left
                more = false;
                break;
            }
            u32x4 qc[C::GR][C::KS];
            uint16_t* wq = stg + wave * (2 * C::UNIT * D);  // this wave's Q tile, then its O tile
            uint16_t* wo = wq + C::UNIT * D;
            if (C::STG) {
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
            us[s] = tok_of(grab());
            load_unit(qr[s], us[s]);

#pragma unroll
            for (int r = 0; r < C::GR; ++r) {
                const int tl = u0 + 16 * r + n;  // token within the chunk
                Pos3 ps;
                if (ROPE) ps = token_pos((uint32_t)(a.g.n_offset + c0 + min(tl, len - 1)), t_lo, a.g);
                float den = 0.0f;
                f32x4 dacc = f32x4{0.f, 0.f, 0.f, 0.f};
                f32x4 acc[C::NT];
#pragma unroll
                for (int T = 0; T < C::NT; ++T) acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
                // relu(Q) of the group (channels past d, loaded from the next
                // row at d = 112, are zeroed), and whether any lane holds a
                // value fp16 cannot carry exactly enough: then every token of
                // the group is scaled by 2^sc, sc = 13 - (exponent of its
                // largest relu(Q) value)
                uint32_t m16 = 0;
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    const bool live = C::DP == D || 32 * ks + 8 * g < D;
                    const uint32_t mk = live ? max_relu_bits8(qc[r][ks]) : 0u;
                    m16 = mk > m16 ? mk : m16;
                }
                // bf16 bit patterns of 2^-6 and 2^14
                const bool odd = m16 != 0 && (m16 < 0x3C80u || m16 >= 0x4680u);
                // (d >= 112: always, without a branch -- a branch inside the
                // k-step loop makes the 768-thread kernel spill registers)
                const bool scaled = C::SLDS || __builtin_amdgcn_ballot_w64(odd) != 0;
                int sc = 0;
                if (scaled) {
                    uint32_t tm = m16;
                    tm = max(tm, (uint32_t)__shfl_xor((int)tm, 16));
                    tm = max(tm, (uint32_t)__shfl_xor((int)tm, 32));
                    sc = tm != 0 ? 13 - ((int)(tm >> 7) - 127) : 0;
                }
                // one 32-channel k-step at a time: its B fragments, then its MFMAs
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
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
                        const float4 za = *(const float4*)(zs + 32 * ks + 8 * g);
                        const float4 zb = *(const float4*)(zs + 32 * ks + 8 * g + 4);
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
                    if (ROPE) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) rotate(x[2 * i], x[2 * i + 1], tab[pair_entry(pr[ks][i], ps)]);
                    }
                    u32x4 hw;
#pragma unroll
                    for (int i = 0; i < 4; ++i) hw[i] = pack_f16(x[2 * i], x[2 * i + 1]);
                    const f16x8 Bq = __builtin_bit_cast(f16x8, hw);
#pragma unroll
                    for (int T = 0; T < C::NT; ++T) {
                        const f16x8 A = C::SLDS ? *(const f16x8*)(st + st_off<C::DP>(16 * T + n, 4 * ks + g))
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
                // undo the scalings: S by 2^-eS, the group's tokens by 2^sc
                const float inv = den > 0.0f ? ldexpf(1.0f / den, eS - sc) : 0.0f;
#pragma unroll
                for (int sp = 0; sp < C::NT / 2; ++sp) {
                    u32x4 o;
                    o[0] = pack_bf16(acc[2 * sp][0] * inv, acc[2 * sp][1] * inv);
                    o[1] = pack_bf16(acc[2 * sp][2] * inv, acc[2 * sp][3] * inv);
                    o[2] = pack_bf16(acc[2 * sp + 1][0] * inv, acc[2 * sp + 1][1] * inv);
                    o[3] = pack_bf16(acc[2 * sp + 1][2] * inv, acc[2 * sp + 1][3] * inv);
                    if (C::STG)
                        *(u32x4*)(wo + stg_off(16 * r + n, 4 * sp + g)) = o;
                    else if (C::DP == D || 32 * sp + 8 * g < D)  // part-lines: let L2 merge them
                        buf_store16(o, Or, (uint32_t)(tl * D + 32 * sp + 8 * g) * 2u);
                }
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
    static constexpr int SMEM_FIXED = (D * D + D + 2 * TT * D + TT) * 4;
};

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void la_apply_f32_kernel(ApplyArgs a) {
    using C = ApplyF32Cfg<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    float* Ss = (float*)smem;        // [D][D]
    float* zs = Ss + D * D;          // [D]
    float* qp = zs + D;              // [TT][D] relu(Q)
    float* qq = qp + C::TT * D;      // [TT][D] RoPE(relu(Q))
    float* dn = qq + C::TT * D;      // [TT]
    float2* tab = (float2*)(smem + C::SMEM_FIXED);

    const int tid = threadIdx.x;
    int bh, p;
    apply_item_of_block(a.P, a.g.BH, bh, p);
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
            for (int c = 0; c < D; ++c) s = fmaf(qp[tid * D + c], zs[c], s);
            dn[tid] = s + a.eps;
        }
        lds_barrier();
        for (int i = tid; i < C::TT * D; i += 256) {
            const int tl = i / D, co = i % D;
            const int tok = t0 + tl;
            if (tok >= c1) continue;
            float s = 0.0f;
            for (int ci = 0; ci < D; ++ci) s = fmaf(qq[tl * D + ci], Ss[ci * D + co], s);
            const float den = dn[tl];
            Oh[(size_t)tok * D + co] = den > 0.0f ? s / den : 0.0f;
        }
    }
}
