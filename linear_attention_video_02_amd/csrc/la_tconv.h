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
    int mtiles, ntiles;     // ceil(M / BM), ceil(D / BN)
    int group;              // token tiles per group of the tile order
};

// 320 output channels x 160 tokens per workgroup (the 720p block at width
// 2240 is 7 x 138 such tiles, no ragged edge), K in stages of 64 channels,
// double-buffered in LDS (120 KB, one workgroup per CU).  8 waves in a 4 x 2
// grid, each 80 channels x 80 tokens = 5 x 5 tiles of v_mfma_f32_16x16x32_bf16
// (100 accumulators in VGPRs): per 32-deep k step a wave reads 10 fragments
// for 25 MFMAs; two waves share each SIMD and hide each other's LDS reads.
struct TconvCfg {
    static constexpr int BN = 320, BM = 160, BK = 64;
    static constexpr int THREADS = 512;
    static constexpr int WN = 5, WM = 5;               // 16 x 16 tiles per wave
    static constexpr int ROWS = BN + BM;               // LDS rows per stage (W, then X)
    static constexpr int STAGE = ROWS * BK;            // bf16 elements per stage
    static constexpr int LDS_BYTES = 2 * STAGE * 2;    // two stages
    static constexpr int XR = 3;                       // X rows per loader thread (last: tid < 256)
};

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
