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
// bf16 operands, fp32 accumulation on v_mfma_f32_16x16x32_bf16, bf16 output.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

struct TconvArgs {
    const uint16_t* X;      // [B][T][P][D] bf16, token-major (frame, then position)
    uint16_t* Y;            // [B][T][P][D] bf16
    const uint16_t* W;      // [3][D][D] bf16, W[k][out][in], k = time offset + 1
    const float* bias;      // [D] fp32 or null
    const uint16_t* cache;  // [B][P][D] bf16: the previous block's last frame
    int T, P, D;
    int M;                  // B * T * P tokens
    int F, S;               // token tile: F = min(T, 8) frames x S positions (tconv_positions)
    int nft, npt;           // ceil(T / F), ceil(P / S)
    int mtiles, ntiles;     // B * nft * npt token tiles, ceil(D / 160) channel tiles
    int gm, gn;             // tile-order group: gm token tiles by gn channel tiles
};

// 160 output channels x 320 tokens per workgroup, the tokens being 8 frames x
// 40 positions (the 720p block, 24 frames x 920 positions at width 2240, is
// 14 x 69 such tiles with no ragged edge).  K runs over 64-channel chunks,
// each taken at the three time offsets in turn (K = 3D).  Per chunk the
// tile's 10-frame union (one frame before, one after) is staged in LDS once
// and read by all three offsets at row shifts of 0, 40 and 80; W slices are
// staged per offset.  Both are double-buffered: 140 KB of LDS, one
// workgroup per CU.  8 waves in a 2 x 4 grid, each 80 channels x 80 tokens =
// 5 x 5 tiles of v_mfma_f32_16x16x32_bf16 (100 accumulators in VGPRs): per
// 32-deep k step a wave reads 10 fragments for 25 MFMAs.
struct TconvCfg {
    static constexpr int BN = 160, BM = 320, BK = 64;
    static constexpr int THREADS = 512;
    static constexpr int WN = 5, WM = 5;                 // 16 x 16 tiles per wave
    static constexpr int FMAX = 8;                       // token tile: F <= 8 frames x S positions
    static constexpr int UROWS = 400;                    // frame-union rows per chunk: (F + 2) S <= 400
    static constexpr int WSTAGE = BN * BK;               // bf16 elements of a W slice
    static constexpr int XSTAGE = UROWS * BK;            // bf16 elements of a union chunk
    static constexpr int LDS_BYTES = (3 * WSTAGE + 2 * XSTAGE) * 2;  // 160 KB, all of it
};

// Positions per token tile for a tile of F frames: the largest multiple of 8
// with F S <= 320 (the tile's rows) and (F + 2) S <= 400 (the frame union's
// rows): 128, 96, 80, 64, 56, 48, 40, 40 for F = 1 .. 8.
inline int tconv_positions(int F) {
    int s = TconvCfg::BM / F;
    const int u = TconvCfg::UROWS / (F + 2);
    if (u < s) s = u;
    return s & ~7;
}

// The cache after a block: its last input frame, X[b][T-1] -> cache[b].
struct TconvCacheArgs {
    const uint16_t* X;
    uint16_t* cache;
    int T, P, D, B;
};

// Launches of the kernels in la_tconv.hip (a translation unit of its own,
// compiled with the MFMA accumulators in VGPRs).  Return the launch status.
hipError_t la_tconv_launch(const TconvArgs& a, hipStream_t st);
hipError_t la_tconv_cache_launch(const TconvCacheArgs& c, hipStream_t st);
