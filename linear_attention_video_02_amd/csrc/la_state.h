// State pass of ReLU linear attention (the two sums of the linear-attention
// equation on the SANA-Video analysis page, section 3.4, in the Eq. 2 form):
//
//   S = sum_j RoPE(relu(K_j))^T V_j   (d x d, fp32)      z = sum_j relu(K_j)   (d, fp32)
//
// Work split: grid (P, B*H).  Workgroup p of head bh reduces the token chunk
// [p*chunk, (p+1)*chunk) to a partial (S_p, z_p) in the workspace.  A second,
// small kernel (la_state_combine_kernel) sums the P partials of each head in
// the fixed order p = 0..P-1, adds the carried state when there is one
// (block-causal mode, Eq. 3 / Algorithm 1) and writes S and z.  No atomics
// and no in-kernel cross-workgroup signalling: the kernel boundary makes the
// partials visible (an in-kernel device-scope fence per workgroup would write
// back and invalidate a whole XCD L2 each time).  Results are bitwise
// reproducible for a given shape.
#pragma once

#include "la_common.h"

struct StateArgs {
    const void* K;
    const void* V;
    float* partial;        // [BH][P][D*D + D]
    int chunk;             // tokens per workgroup
    int P;                 // workgroups per (batch, head)
    LaGeom g;
};

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

// Stage 2: grid (ceil(E4 / 256), B*H), one float4 of (S, z) per thread.  Sums
// the P partials in the fixed order p = 0..P-1 (eight partials' loads in
// flight before they are added), then adds the carry: S_b = carry + sum_p S_p.
template <int D>
__global__ __launch_bounds__(256) void la_state_combine_kernel(CombineArgs a) {
    constexpr int E = D * D + D;
    constexpr int E4 = E / 4;  // S and z regions both hold whole float4s (D % 4 == 0)
    const int f = blockIdx.x * 256 + threadIdx.x;
    const int bh = blockIdx.y;
    if (f >= E4) return;
    const float4* part = (const float4*)(a.partial + (size_t)bh * a.P * E);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int p = 0;
    for (; p + 8 <= a.P; p += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(p + u) * E4 + f];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
        }
    }
    {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (p + u < a.P) v[u] = part[(size_t)(p + u) * E4 + f];
#pragma unroll
        for (int u = 0; u < 8; ++u)
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
// bf16 inputs: MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation.
//
// Per 64-token tile: every thread loads 16-byte pieces (8 channels of one
// token) of K and V, coalesced.  K gets relu, the z partial (un-rotated),
// RoPE at the token's global grid position, and bf16 rounding; K and V are
// then written to LDS TRANSPOSED (row = channel, 64 tokens per row) so that
// an MFMA operand -- 8 consecutive tokens of one channel -- is one 16-byte
// LDS read.  8-token column blocks are XOR-swizzled by channel block to
// spread LDS banks.  MFMA: C[c_in][c_out] += A[c_in][tok] B[tok][c_out] with
// A = RoPE(relu K)^T, B = V.
//   d = 32, 64: wave w takes tokens 16w..16w+15 of the tile and all d x d
//               outputs; the 4 waves are summed in LDS at the end in the
//               fixed order (w0 + w1) + (w2 + w3).
//   d = 128:    wave w takes key channels 32w..32w+31, all 64 tokens.
// ---------------------------------------------------------------------------
template <int D>
struct StateBf16Cfg {
    static constexpr int CH = D / 8;          // 16-byte pieces per token row
    static constexpr int ROWS = 256 / CH;     // token rows per load pass
    static constexpr int TT = 64;             // tokens per tile
    static constexpr int LP = TT / ROWS;      // load passes per tile
    static constexpr int PITCH = TT + 8;      // LDS row pitch (bf16) of the transposed tiles
    static constexpr bool SPLIT_TOK = D <= 64;
    static constexpr int NI = SPLIT_TOK ? D / 32 : 1;   // key-channel tiles per wave
    static constexpr int NJ = D / 32;                   // value-channel tiles per wave
    static constexpr int KSTEPS = SPLIT_TOK ? 1 : 4;    // 16-token steps per wave per tile
    static constexpr int STAGE_BYTES = 2 * D * PITCH * 2;
    static constexpr int RED_BYTES = SPLIT_TOK ? 64 * NI * NJ * 16 * 4 : 0;
    static constexpr int ZRED_BYTES = 256 * 8 * 4;
    static constexpr int m1 = STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES;
    static constexpr int SMEM_FIXED = m1 > ZRED_BYTES ? m1 : ZRED_BYTES;
};

__device__ __forceinline__ int swz_col(int c, int tok) {
    return (((tok >> 3) ^ ((c >> 3) & 7)) << 3) | (tok & 7);
}

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void la_state_bf16_kernel(StateArgs a) {
    using C = StateBf16Cfg<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* ks = (uint16_t*)smem;
    uint16_t* vs = ks + D * C::PITCH;
    float2* tab = (float2*)(smem + C::SMEM_FIXED);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = blockIdx.x, bh = blockIdx.y;
    const int ntok = a.g.ntok;
    const int c0 = p * a.chunk;
    const int c1 = min(c0 + a.chunk, ntok);
    const size_t head = (size_t)bh * ntok * D;
    const uint16_t* Kh = (const uint16_t*)a.K + head;
    const uint16_t* Vh = (const uint16_t*)a.V + head;
    const int cc = tid % C::CH, trow = tid / C::CH;

    u32x4 kr[C::LP], vr[C::LP];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int j = 0; j < C::LP; ++j) {
            int tok = t0 + trow + j * C::ROWS;
            if (tok < c1) {
                kr[j] = *(const u32x4*)(Kh + (size_t)tok * D + 8 * cc);
                vr[j] = *(const u32x4*)(Vh + (size_t)tok * D + 8 * cc);
            } else {
                kr[j] = u32x4{0u, 0u, 0u, 0u};
                vr[j] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    if (c0 < c1) load_tile(c0);

    int t_lo = 0;
    PairRef pr[4];
    if (ROPE) {
        const int cl = c1 > c0 ? c1 - 1 : c0;
        t_lo = (int)fdiv((uint32_t)(a.g.n_offset + c0), a.g.div_hw);
        int nt = (int)fdiv((uint32_t)(a.g.n_offset + cl), a.g.div_hw) - t_lo + 1;
        build_rope_table(tab, t_lo, nt, a.g);
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = pair_ref(4 * cc + i, nt, a.g);
    }

    float zp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zp[e] = 0.0f;
    f32x16 acc[C::NI][C::NJ];
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int m = lane & 31, gq = lane >> 5;

    for (int t0 = c0; t0 < c1; t0 += C::TT) {
        __syncthreads();  // LDS tiles free (and RoPE table complete)
#pragma unroll
        for (int j = 0; j < C::LP; ++j) {
            const int tl = trow + j * C::ROWS;
            float x[8];
            const uint32_t w4[4] = {kr[j][0], kr[j][1], kr[j][2], kr[j][3]};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = fmaxf(bf_lo(w4[i]), 0.0f);
                x[2 * i + 1] = fmaxf(bf_hi(w4[i]), 0.0f);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) zp[e] += x[e];
            if (ROPE) {
                int tok = min(t0 + tl, c1 - 1);
                Pos3 ps = token_pos((uint32_t)(a.g.n_offset + tok), t_lo, a.g);
#pragma unroll
                for (int i = 0; i < 4; ++i) rotate(x[2 * i], x[2 * i + 1], tab[pair_entry(pr[i], ps)]);
            }
            uint32_t kw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) kw[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 8 * cc + e;
                const int col = swz_col(c, tl);
                ks[c * C::PITCH + col] = (uint16_t)(kw[e >> 1] >> ((e & 1) * 16));
                vs[c * C::PITCH + col] = (uint16_t)(vr[j][e >> 1] >> ((e & 1) * 16));
            }
        }
        __syncthreads();
        if (t0 + C::TT < c1) load_tile(t0 + C::TT);

#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            const int kb = C::SPLIT_TOK ? 2 * wave + gq : 2 * s + gq;  // 8-token block
            bf16x8 A[C::NI], Bv[C::NJ];
#pragma unroll
            for (int i = 0; i < C::NI; ++i) {
                const int c = 32 * (C::SPLIT_TOK ? i : wave) + m;
                A[i] = *(const bf16x8*)(ks + c * C::PITCH + ((kb ^ ((c >> 3) & 7)) << 3));
            }
#pragma unroll
            for (int j = 0; j < C::NJ; ++j) {
                const int c = 32 * j + m;
                Bv[j] = *(const bf16x8*)(vs + c * C::PITCH + ((kb ^ ((c >> 3) & 7)) << 3));
            }
#pragma unroll
            for (int i = 0; i < C::NI; ++i)
#pragma unroll
                for (int j = 0; j < C::NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], Bv[j], acc[i][j], 0, 0, 0);
        }
    }

    // ---- fold the waves (d <= 64): fixed order (w0 + w1) + (w2 + w3) ----
    float* red = (float*)smem;
    constexpr int NACC = C::NI * C::NJ * 16;
    if (C::SPLIT_TOK) {
        auto put = [&]() {
#pragma unroll
            for (int i = 0; i < C::NI; ++i)
#pragma unroll
                for (int j = 0; j < C::NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[((i * C::NJ + j) * 16 + r) * 64 + lane] = acc[i][j][r];
        };
        auto add = [&]() {
#pragma unroll
            for (int i = 0; i < C::NI; ++i)
#pragma unroll
                for (int j = 0; j < C::NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * C::NJ + j) * 16 + r) * 64 + lane];
        };
        static_assert(NACC * 64 * 4 <= C::SMEM_FIXED, "reduction buffer");
        __syncthreads();
        if (wave == 1) put();
        __syncthreads();
        if (wave == 0) add();
        __syncthreads();
        if (wave == 3) put();
        __syncthreads();
        if (wave == 2) add();
        __syncthreads();
        if (wave == 2) put();
        __syncthreads();
        if (wave == 0) add();
    }

    // ---- write this workgroup's partial ----
    constexpr int E = D * D + D;
    float* part = a.partial + ((size_t)bh * a.P + p) * E;
    if (!C::SPLIT_TOK || wave == 0) {
#pragma unroll
        for (int i = 0; i < C::NI; ++i)
#pragma unroll
            for (int j = 0; j < C::NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * (C::SPLIT_TOK ? i : wave) + 8 * (r >> 2) + 4 * gq + (r & 3);
                    const int col = 32 * j + m;
                    part[row * D + col] = acc[i][j][r];
                }
    }
    // ---- z partial: threads sharing a channel block, summed in thread order ----
    __syncthreads();
    float* zr = (float*)smem;
#pragma unroll
    for (int e = 0; e < 8; ++e) zr[tid * 8 + e] = zp[e];
    __syncthreads();
    if (tid < D) {
        float s = 0.0f;
        for (int r = 0; r < C::ROWS; ++r) s += zr[((tid >> 3) + C::CH * r) * 8 + (tid & 7)];
        part[D * D + tid] = s;
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
    const int p = blockIdx.x, bh = blockIdx.y;
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
        __syncthreads();
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
        __syncthreads();
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
    float* part = a.partial + ((size_t)bh * a.P + p) * E;
#pragma unroll
    for (int j = 0; j < C::NE; ++j) part[tid + 256 * j] = acc[j];
    if (tid < D) part[D * D + tid] = zacc;
}
