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
    LaGeom g;
};

// ---------------------------------------------------------------------------
// bf16: MFMA v_mfma_f32_16x16x32_bf16 with C = S^T . RoPE(relu Q)^T, so that
// every accumulator a lane holds belongs to one token (column n = lane % 16)
// and the B operand -- 8 consecutive channels of one token -- is a plain
// 16-byte load of Q.  S^T is held in registers for the whole workgroup as
// bf16 hi + lo parts (S = hi + lo to ~2^-17), so the product carries only the
// bf16 rounding of RoPE(relu Q).
//
// Lane (n = lane % 16, g = lane / 16) handles token n of a 16-token group and
// the key channels 32*ks + 8*g .. +7, ks = 0 .. d/32 - 1.  Output tile T (16
// value channels) row 4g+i maps to value channel 32*(T/2) + 8g + 4*(T%2) + i,
// so a lane ends with 8 consecutive output channels per pair of tiles: one
// 16-byte store each.  The denominator is summed over the 4 lanes of a token
// with two cross-lane xors.
// Each wave takes GR consecutive 16-token groups per iteration and prefetches
// the next iteration's Q while computing.
// ---------------------------------------------------------------------------
template <int D>
struct ApplyBf16Cfg {
    static constexpr int KS = D / 32;   // 32-channel k-steps
    static constexpr int NT = D / 16;   // 16-channel output tiles
    static constexpr int GR = D <= 64 ? 2 : 1;   // 16-token groups per wave iteration
    static constexpr int TOK_ITER = 4 * 16 * GR; // tokens per workgroup iteration
};

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void la_apply_bf16_kernel(ApplyArgs a) {
    using C = ApplyBf16Cfg<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    float2* tab = (float2*)smem;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int p = blockIdx.x, bh = blockIdx.y;
    const int ntok = a.g.ntok;
    const int c0 = p * a.chunk;
    const int c1 = min(c0 + a.chunk, ntok);
    const size_t head = (size_t)bh * ntok * D;
    const uint16_t* Qh = (const uint16_t*)a.Q + head;
    uint16_t* Oh = (uint16_t*)a.O + head;

    // first iteration's loads go out before the prologue work
    u32x4 qn[C::GR][C::KS];
    auto load_iter = [&](int t0) {
#pragma unroll
        for (int r = 0; r < C::GR; ++r) {
            const int tok = t0 + 16 * r + n;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                if (tok < c1)
                    qn[r][ks] = *(const u32x4*)(Qh + (size_t)tok * D + 32 * ks + 8 * g);
                else
                    qn[r][ks] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    const int tw0 = c0 + wave * 16 * C::GR;
    load_iter(tw0);

    // S^T fragments (hi/lo bf16) and this lane's z entries
    bf16x8 Ahi[C::NT][C::KS], Alo[C::NT][C::KS];
    const float* Sh = a.S + (size_t)bh * D * D;
#pragma unroll
    for (int T = 0; T < C::NT; ++T) {
        const int co = 32 * (T >> 1) + 8 * (n >> 2) + 4 * (T & 1) + (n & 3);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float s = Sh[(32 * ks + 8 * g + e) * D + co];
                const __bf16 hi = (__bf16)s;
                Ahi[T][ks][e] = hi;
                Alo[T][ks][e] = (__bf16)(s - (float)hi);
            }
        }
    }
    float zr[C::KS][8];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) zr[ks][e] = a.z[(size_t)bh * D + 32 * ks + 8 * g + e];

    int t_lo = 0, nt = 1;
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
        __syncthreads();
    }

    for (int t0 = tw0; t0 < c1; t0 += C::TOK_ITER) {
        u32x4 qc[C::GR][C::KS];
#pragma unroll
        for (int r = 0; r < C::GR; ++r)
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) qc[r][ks] = qn[r][ks];
        if (t0 + C::TOK_ITER < c1) load_iter(t0 + C::TOK_ITER);

#pragma unroll
        for (int r = 0; r < C::GR; ++r) {
            const int tok = t0 + 16 * r + n;
            Pos3 ps;
            if (ROPE) ps = token_pos((uint32_t)(a.g.n_offset + min(tok, c1 - 1)), t_lo, a.g);
            float den = 0.0f;
            bf16x8 Bq[C::KS];
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[2 * i] = fmaxf(bf_lo(qc[r][ks][i]), 0.0f);
                    x[2 * i + 1] = fmaxf(bf_hi(qc[r][ks][i]), 0.0f);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) den = fmaf(x[e], zr[ks][e], den);
                if (ROPE) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const PairRef pr = pair_ref(16 * ks + 4 * g + i, nt, a.g);
                        rotate(x[2 * i], x[2 * i + 1], tab[pair_entry(pr, ps)]);
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) Bq[ks][e] = (__bf16)x[e];
            }
            f32x4 acc[C::NT];
#pragma unroll
            for (int T = 0; T < C::NT; ++T) acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
                for (int T = 0; T < C::NT; ++T) {
                    acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ahi[T][ks], Bq[ks], acc[T], 0, 0, 0);
                    acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Alo[T][ks], Bq[ks], acc[T], 0, 0, 0);
                }
            den += __shfl_xor(den, 16);
            den += __shfl_xor(den, 32);
            den += a.eps;
            const float inv = den > 0.0f ? 1.0f / den : 0.0f;
            if (tok < c1) {
#pragma unroll
                for (int s = 0; s < C::NT / 2; ++s) {
                    u32x4 o;
                    o[0] = pack_bf16(acc[2 * s][0] * inv, acc[2 * s][1] * inv);
                    o[1] = pack_bf16(acc[2 * s][2] * inv, acc[2 * s][3] * inv);
                    o[2] = pack_bf16(acc[2 * s + 1][0] * inv, acc[2 * s + 1][1] * inv);
                    o[3] = pack_bf16(acc[2 * s + 1][2] * inv, acc[2 * s + 1][3] * inv);
                    *(u32x4*)(Oh + (size_t)tok * D + 32 * s + 8 * g) = o;
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
    const int p = blockIdx.x, bh = blockIdx.y;
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
        __syncthreads();
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
        __syncthreads();
        if (tid < C::TT) {
            float s = 0.0f;
            for (int c = 0; c < D; ++c) s = fmaf(qp[tid * D + c], zs[c], s);
            dn[tid] = s + a.eps;
        }
        __syncthreads();
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
