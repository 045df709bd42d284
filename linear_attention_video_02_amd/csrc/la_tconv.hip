// Kernels of the block-causal temporal convolution (declared with their
// arguments in la_tconv.h).  Built as a translation unit of its own so that
// the MFMA accumulators can be kept in VGPRs (-amdgpu-mfma-vgpr-form): with
// them in AGPRs the compiler copied accumulators around every MFMA.
#include "la_common.h"
#include "la_tconv.h"

// Element offset of (row, 16-byte chunk c) in a stage of 64-wide bf16 rows:
// chunk c of row r is stored at c ^ (r & 7), so fragment reads (16 rows at one
// chunk) and the loaders' writes (8 whole rows) spread over all banks.
__device__ __forceinline__ int tc_off(int row, int c) { return row * 64 + ((c ^ (row & 7)) << 3); }

__global__ __launch_bounds__(TconvCfg::THREADS) void la_tconv_bf16_kernel(TconvArgs a) {
    using C = TconvCfg;
    extern __shared__ __align__(16) uint16_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // Loader role: thread (lr, lc) = (tid / 8, tid % 8) loads 16-byte chunk
    // lc of W rows lr + 64 j (j < 5) and X rows lr + 64 j (j < 2, and j = 2
    // for lr < 32, i.e. waves 0-3).  Byte offsets of each row's source per
    // segment; kOob (past every buffer's range) reads as zeros: rows past M,
    // the zero padding frame, channels past D.  Segment 0 of a block's first
    // frame reads the cache.
    constexpr uint32_t kOob = 0x80000000u;
    const BufRsrc rX = make_rsrc(a.X, (uint32_t)((size_t)a.M * D * 2));
    const BufRsrc rC = make_rsrc(a.cache, (uint32_t)((size_t)(a.M / TP) * P * D * 2));
    const BufRsrc rW = make_rsrc(a.W, (uint32_t)((size_t)3 * D * D * 2));
    const int lr = tid >> 3, lc = tid & 7;
    const bool third = wave < 4;  // loads X row lr + 128
    uint32_t xo0[C::XR], xo1[C::XR], xo2[C::XR], co0[C::XR], wo[C::BN / 64];
    bool first_rows = false;
#pragma unroll
    for (int j = 0; j < C::XR; ++j) {
        const int m = m0 + lr + 64 * j;
        const bool mv = m < a.M && (j < 2 || third);
        const int b = m / TP, rem = m - b * TP;
        const int f = rem / P, p = rem - f * P;
        const uint32_t xm = (uint32_t)m * (uint32_t)D * 2u + 16u * lc;
        const uint32_t pd = (uint32_t)P * (uint32_t)D * 2u;
        xo0[j] = (mv && f > 0) ? xm - pd : kOob;
        co0[j] = (mv && f == 0) ? ((uint32_t)(b * P + p) * (uint32_t)D * 2u + 16u * lc) : kOob;
        xo1[j] = mv ? xm : kOob;
        xo2[j] = (mv && f + 1 < a.T) ? xm + pd : kOob;
        first_rows |= mv && f == 0;
    }
#pragma unroll
    for (int j = 0; j < C::BN / 64; ++j) {
        const int n = n0 + lr + 64 * j;
        wo[j] = n < D ? (uint32_t)n * (uint32_t)D * 2u + 16u * lc : kOob;
    }
    // wave-uniform: does any X row this wave loads start a block?
    first_rows = __builtin_amdgcn_ballot_w64(first_rows) != 0;
    const int kpd = D / C::BK;  // stages per segment
    const int KT = 3 * kpd;
    u32x4 rw[C::BN / 64], rx[C::XR];
    auto load_stage = [&](int kt) {
        const int seg = kt / kpd;
        const uint32_t kb = (uint32_t)(kt - seg * kpd) * (C::BK * 2);
        const uint32_t wk = (uint32_t)seg * (uint32_t)D * (uint32_t)D * 2u + kb;
#pragma unroll
        for (int j = 0; j < C::BN / 64; ++j) rw[j] = buf_load16(rW, wo[j] + wk);
#pragma unroll
        for (int j = 0; j < C::XR; ++j) {
            if (j == 2 && !third) break;
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
        uint16_t* st = lds + buf * C::STAGE;
#pragma unroll
        for (int j = 0; j < C::BN / 64; ++j) *(u32x4*)(st + tc_off(lr + 64 * j, lc)) = rw[j];
#pragma unroll
        for (int j = 0; j < C::XR; ++j) {
            if (j == 2 && !third) break;
            *(u32x4*)(st + tc_off(C::BN + lr + 64 * j, lc)) = rx[j];
        }
    };

    // Compute role: wave (wn, wm) owns channels 80 wn .. +79 and tokens
    // 80 wm .. +79.  Fragment lane layout (16 x 16 x 32): lane l reads row
    // l % 16 of a 16-row block at k chunk l / 16 (8 consecutive k).
    const int wn = wave & 3, wm = wave >> 2;
    const int fr = lane & 15, fc = lane >> 4;
    f32x4 acc[C::WN][C::WM];
#pragma unroll
    for (int i = 0; i < C::WN; ++i)
#pragma unroll
        for (int j = 0; j < C::WM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    load_stage(0);
    store_stage(0);
    if (KT > 1) load_stage(1);
    lds_barrier();
    for (int kt = 0; kt < KT; ++kt) {
        const uint16_t* st = lds + (kt & 1) * C::STAGE;
#pragma unroll
        for (int ks = 0; ks < C::BK / 32; ++ks) {
            bf16x8 xf[C::WM];
#pragma unroll
            for (int j = 0; j < C::WM; ++j)
                xf[j] = *(const bf16x8*)(st + tc_off(C::BN + 80 * wm + 16 * j + fr, 4 * ks + fc));
#pragma unroll
            for (int i = 0; i < C::WN; ++i) {
                const bf16x8 wf = *(const bf16x8*)(st + tc_off(80 * wn + 16 * i + fr, 4 * ks + fc));
#pragma unroll
                for (int j = 0; j < C::WM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[j], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < KT) store_stage((kt + 1) & 1);  // its readers passed the last barrier
        if (kt + 2 < KT) load_stage(kt + 2);          // lands during the next stage
        lds_barrier();
    }

    // Epilogue: lane holds C[n][m] for token m = .. + lane % 16 and channels
    // n = .. + 4 (lane / 16) + (0..3): 4 consecutive channels of one token.
#pragma unroll
    for (int j = 0; j < C::WM; ++j) {
        const int m = m0 + 80 * wm + 16 * j + fr;
        if (m >= a.M) continue;
#pragma unroll
        for (int i = 0; i < C::WN; ++i) {
            const int n = n0 + 80 * wn + 16 * i + 4 * fc;
            if (n >= D) continue;
            const size_t o = (size_t)m * D + n;
            const uint2 xv = *(const uint2*)(a.X + o);
            float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (a.bias) bv = *(const float4*)(a.bias + n);
            const float y0 = bf_lo(xv.x) + acc[i][j][0] + bv.x;
            const float y1 = bf_hi(xv.x) + acc[i][j][1] + bv.y;
            const float y2 = bf_lo(xv.y) + acc[i][j][2] + bv.z;
            const float y3 = bf_hi(xv.y) + acc[i][j][3] + bv.w;
            *(uint2*)(a.Y + o) = make_uint2(pack_bf16(y0, y1), pack_bf16(y2, y3));
        }
    }
}

__global__ __launch_bounds__(256) void la_tconv_cache_kernel(TconvCacheArgs a) {
    const size_t frame = (size_t)a.P * a.D / 8;  // 16-byte pieces per frame
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= frame * a.B) return;
    const size_t b = i / frame, r = i - b * frame;
    const u32x4* src = (const u32x4*)(a.X + ((size_t)b * a.T + a.T - 1) * a.P * a.D);
    ((u32x4*)(a.cache + b * a.P * a.D))[r] = src[r];
}

hipError_t la_tconv_launch(const TconvArgs& a, hipStream_t st) {
    static bool attr_set = false;  // the attribute is per function; setting it twice is harmless
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute((const void*)la_tconv_bf16_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, TconvCfg::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(la_tconv_bf16_kernel, dim3(a.mtiles * a.ntiles), dim3(TconvCfg::THREADS),
                       TconvCfg::LDS_BYTES, st, a);
    return hipGetLastError();
}

hipError_t la_tconv_cache_launch(const TconvCacheArgs& c, hipStream_t st) {
    const size_t pieces = (size_t)c.B * c.P * c.D / 8;
    hipLaunchKernelGGL(la_tconv_cache_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st, c);
    return hipGetLastError();
}
