// Block-causal temporal convolution of the Mix-FFN with its shortcut (the
// SANA-Video analysis page, section 3.4, "Spatial-Temporal Mix-FFN" and
// "Block Causal Mix-FFN"):
//
//   Y[f] = X[f] + W_0 X[f-1] + W_1 X[f] + W_2 X[f+1] (+ bias),
//
// per spatial position, with X[-1] the cached last frame of the previous
// block and X[T] the zero padding frame.  Each W_k is D x D (row = output
// channel), so the operation is a GEMM with K = 3D whose A rows are each
// token's previous, own and next frame:
//
//   C[n][m] = sum_{k, i} W_k[n][i] X_k[m][i],   Y[m][n] = X[m][n] + C[n][m] (+ bias[n])
//
// bf16 operands, fp32 accumulation on v_mfma_f32_32x32x16_bf16, bf16 output.
#pragma once

#include "la_common.h"

struct TconvArgs {
    const uint16_t* X;      // [B][T][P][D] bf16, token-major (frame, then position)
    uint16_t* Y;            // [B][T][P][D] bf16
    const uint16_t* W;      // [3][D][D] bf16, W[k][out][in], k = time offset + 1
    const float* bias;      // [D] fp32 or null
    const uint16_t* cache;  // [B][P][D] bf16: the previous block's last frame
    int T, P, D;
    int M;                  // B * T * P tokens
    int mtiles, ntiles;     // ceil(M / 128), ceil(D / 128)
    int group;              // token tiles per group of the tile order
};

// 128 (output channels) x 128 (tokens) per workgroup, K in stages of 64
// channels; 4 waves, each 64 x 64 = 2 x 2 MFMA tiles of 32 x 32.
struct TconvCfg {
    static constexpr int BN = 128, BM = 128, BK = 64;
    static constexpr int THREADS = 256;
    static constexpr int TILE = 128 * BK;  // bf16 elements of one operand tile
};

// Element offset of (row, 16-byte chunk c) in a [128][64] bf16 LDS tile:
// chunk c of row r is stored at c ^ (r & 7), so the 32 rows an MFMA operand
// read touches at one chunk fall in 8 different chunk slots.
__device__ __forceinline__ int tc_off(int row, int c) { return row * 64 + ((c ^ (row & 7)) << 3); }

__global__ __launch_bounds__(TconvCfg::THREADS) void la_tconv_bf16_kernel(TconvArgs a) {
    using C = TconvCfg;
    __shared__ __align__(16) uint16_t lds[2][2][C::TILE];  // [buffer][W, X]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Tile order.  Workgroup b runs on XCD b % 8; the XCD's k-th workgroup
    // takes tile v = (b % 8) * (tiles / 8) + k, so each XCD works through a
    // contiguous range of v.  v walks `group` token tiles by all channel
    // tiles, so the workgroups resident on one XCD at a time share their X
    // and W slices in that XCD's L2.  (The last tiles % 8 workgroups keep
    // v = b.)  Both steps are bijections onto [0, tiles).
    int mt, nt;
    {
        const int tiles = a.mtiles * a.ntiles, per = tiles >> 3;
        int v = blockIdx.x;
        if (v < per * 8) v = (v & 7) * per + (v >> 3);
        const int span = a.group * a.ntiles, g = v / span, first = g * a.group;
        const int gm = min(a.mtiles - first, a.group), r = v - g * span;
        mt = first + r % gm;
        nt = r / gm;
    }
    const int m0 = mt * C::BM, n0 = nt * C::BN;
    const int D = a.D, P = a.P, TP = a.T * a.P;

    // Loader role: rows lr + 32 j (j = 0..3) of both tiles, 16-byte chunk lc.
    // Byte offsets of each row's source per segment; kOob (past every
    // buffer's range) reads as zeros: rows past M, the zero padding frame,
    // channels past D.  Segment 0 of a block's first frame reads the cache.
    constexpr uint32_t kOob = 0x80000000u;
    const BufRsrc rX = make_rsrc(a.X, (uint32_t)((size_t)a.M * D * 2));
    const BufRsrc rC = make_rsrc(a.cache, (uint32_t)((size_t)(a.M / TP) * P * D * 2));
    const BufRsrc rW = make_rsrc(a.W, (uint32_t)((size_t)3 * D * D * 2));
    const int lr = tid >> 3, lc = tid & 7;
    uint32_t xo0[4], xo1[4], xo2[4], co0[4], wo[4];
    bool first_rows = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = m0 + lr + 32 * j;
        const bool mv = m < a.M;
        const int b = m / TP, rem = m - b * TP;
        const int f = rem / P, p = rem - f * P;
        const uint32_t xm = (uint32_t)m * (uint32_t)D * 2u + 16u * lc;
        const uint32_t pd = (uint32_t)P * (uint32_t)D * 2u;
        xo0[j] = (mv && f > 0) ? xm - pd : kOob;
        co0[j] = (mv && f == 0) ? ((uint32_t)(b * P + p) * (uint32_t)D * 2u + 16u * lc) : kOob;
        xo1[j] = mv ? xm : kOob;
        xo2[j] = (mv && f + 1 < a.T) ? xm + pd : kOob;
        first_rows |= mv && f == 0;
        const int n = n0 + lr + 32 * j;
        wo[j] = n < D ? (uint32_t)n * (uint32_t)D * 2u + 16u * lc : kOob;
    }
    // wave-uniform: does any row of this wave's share start a block?
    first_rows = __builtin_amdgcn_ballot_w64(first_rows) != 0;
    const int kpd = D / C::BK;  // stages per segment
    const int KT = 3 * kpd;
    u32x4 rw[4], rx[4];
    auto load_stage = [&](int kt) {
        const int seg = kt / kpd;
        const uint32_t kb = (uint32_t)(kt - seg * kpd) * (C::BK * 2);
        const uint32_t wk = (uint32_t)seg * (uint32_t)D * (uint32_t)D * 2u + kb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rw[j] = buf_load16(rW, wo[j] + wk);
            if (seg == 1) {
                rx[j] = buf_load16(rX, xo1[j] + kb);
            } else if (seg == 2) {
                rx[j] = buf_load16(rX, xo2[j] + kb);
            } else {
                rx[j] = buf_load16(rX, xo0[j] + kb);
                if (first_rows) rx[j] |= buf_load16(rC, co0[j] + kb);
            }
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *(u32x4*)(&lds[buf][0][tc_off(lr + 32 * j, lc)]) = rw[j];
            *(u32x4*)(&lds[buf][1][tc_off(lr + 32 * j, lc)]) = rx[j];
        }
    };

    // Compute role: wave (wn, wm) owns channels wn*64 .. +63, tokens wm*64 .. +63.
    const int wn = wave & 1, wm = wave >> 1;
    const int fr = lane & 31, fk = lane >> 5;  // fragment row, k half
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    load_stage(0);
    store_stage(0);
    lds_barrier();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load_stage(kt + 1);  // in flight during this stage's MFMAs
#pragma unroll
        for (int ks = 0; ks < C::BK / 16; ++ks) {
            bf16x8 A[2], Bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                A[i] = *(const bf16x8*)(&lds[buf][0][tc_off(64 * wn + 32 * i + fr, 2 * ks + fk)]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                Bf[j] = *(const bf16x8*)(&lds[buf][1][tc_off(64 * wm + 32 * j + fr, 2 * ks + fk)]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], Bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) store_stage(buf ^ 1);
        lds_barrier();
    }

    // Epilogue: lane holds C[n][m] for token m = ...(lane & 31) and channels
    // n = 8 q + 4 (lane >> 5) + (0..3), q = 0..3: 4 consecutive channels.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int m = m0 + 64 * wm + 32 * j + fr;
            if (m >= a.M) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + 64 * wn + 32 * i + 8 * q + 4 * fk;
                if (n >= D) continue;
                const size_t o = (size_t)m * D + n;
                const uint2 xv = *(const uint2*)(a.X + o);
                float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (a.bias) bv = *(const float4*)(a.bias + n);
                const float y0 = bf_lo(xv.x) + acc[i][j][4 * q + 0] + bv.x;
                const float y1 = bf_hi(xv.x) + acc[i][j][4 * q + 1] + bv.y;
                const float y2 = bf_lo(xv.y) + acc[i][j][4 * q + 2] + bv.z;
                const float y3 = bf_hi(xv.y) + acc[i][j][4 * q + 3] + bv.w;
                *(uint2*)(a.Y + o) = make_uint2(pack_bf16(y0, y1), pack_bf16(y2, y3));
            }
        }
}

// The cache after a block: its last input frame, X[b][T-1] -> cache[b].
struct TconvCacheArgs {
    const uint16_t* X;
    uint16_t* cache;
    int T, P, D, B;
};

__global__ __launch_bounds__(256) void la_tconv_cache_kernel(TconvCacheArgs a) {
    const size_t frame = (size_t)a.P * a.D / 8;  // 16-byte pieces per frame
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= frame * a.B) return;
    const size_t b = i / frame, r = i - b * frame;
    const u32x4* src = (const u32x4*)(a.X + ((size_t)b * a.T + a.T - 1) * a.P * a.D);
    ((u32x4*)(a.cache + b * a.P * a.D))[r] = src[r];
}
