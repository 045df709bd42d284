// Kernels of the block-causal temporal convolution (declared with their
// arguments in la_tconv.h).  Built as a translation unit of its own so that
// the MFMA accumulators can be kept in VGPRs (-amdgpu-mfma-vgpr-form): with
// them in AGPRs the compiler copied accumulators around every MFMA.
#include "la_common.h"
#include "la_tconv.h"

// Element offset of (row, 16-byte chunk c) in LDS tiles of 64-wide bf16 rows:
// chunk c of row r is stored at c ^ (r & 7), so fragment reads (16 rows at one
// chunk) and the loaders' writes (8 whole rows) spread over all banks.
__device__ __forceinline__ int tc_off(int row, int c) { return row * 64 + ((c ^ (row & 7)) << 3); }

__global__ __launch_bounds__(TconvCfg::THREADS) void la_tconv_bf16_kernel(TconvArgs a) {
    using C = TconvCfg;
    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t* const wbuf0 = lds;                          // W slice of a stage, two buffers
    uint16_t* const xbuf0 = lds + 2 * C::WSTAGE;          // frame union of a chunk, two buffers

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Tile order.  Workgroup b runs on XCD b % 8; the XCD's k-th workgroup
    // takes tile v = (b % 8) * (tiles / 8) + k, so each XCD works through a
    // contiguous range of v (the last tiles % 8 workgroups keep v = b).  v
    // walks groups of GM token tiles; inside one, sub-groups of GN channel
    // tiles, token tile fastest: the workgroups resident on one XCD at a time
    // share X and W slices in its L2.  Every step is a bijection onto [0, tiles).
    int mt, nt;
    {
        const int tiles = a.mtiles * a.ntiles, per = tiles >> 3;
        int v = blockIdx.x;
        if (v < per * 8) v = (v & 7) * per + (v >> 3);
        const int gi = v / (a.gm * a.ntiles), rem = v - gi * (a.gm * a.ntiles);
        const int gm = min(a.gm, a.mtiles - gi * a.gm);
        const int sub = rem / (gm * a.gn), rem2 = rem - sub * (gm * a.gn);
        mt = gi * a.gm + rem2 % gm;
        nt = sub * a.gn + rem2 / gm;
    }
    // Token tile mt: frames f0 .. f0 + F - 1 by positions p0 .. p0 + 39 of batch
    // element bb; tile row r = 40 i + q holds token (f0 + i, p0 + q).  Its
    // frame union, frames f0 - 1 .. f0 + F, is staged per 64-channel chunk as
    // union rows u = 40 i' + q (frame f0 - 1 + i'), so time offset o in {-1, 0, 1}
    // of tile row r is union row r + 40 (o + 1).
    const int F = a.F, D = a.D, P = a.P, T = a.T;
    const int pt = mt % a.npt, ft = (mt / a.npt) % a.nft, bb = mt / (a.npt * a.nft);
    const int f0 = ft * F, p0 = pt * C::S, n0 = nt * C::BN;

    // Loaders.  Thread (lr, lc) = (tid / 8, tid % 8) moves 16-byte chunk lc of
    // W rows lr + 64 j (j < 2; j = 2 for waves 0-3) and of union rows
    // 128 s + lr + 64 j in piece s (j < 2; j = 2 in piece 2 for waves 0-1,
    // rows 384..399).  kOob (past every buffer's range) reads as zeros:
    // channels past D, positions past P, frames past the block (its zero
    // padding frame) and union rows past frame f0 + F.  Union frame f0 - 1 = -1
    // (a block's first tile) reads the cache.
    constexpr uint32_t kOob = 0x80000000u;
    const BufRsrc rX = make_rsrc(a.X, (uint32_t)((size_t)a.M * D * 2));
    const BufRsrc rC = make_rsrc(a.cache, (uint32_t)((size_t)(a.M / (T * P)) * P * D * 2));
    const BufRsrc rW = make_rsrc(a.W, (uint32_t)((size_t)3 * D * D * 2));
    const int lr = tid >> 3, lc = tid & 7;
    uint32_t wo[3], xo[7], co = kOob;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int n = n0 + lr + 64 * j;
        wo[j] = (n < D && lr + 64 * j < C::BN) ? (uint32_t)n * (uint32_t)D * 2u + 16u * lc : kOob;
    }
#pragma unroll
    for (int k = 0; k < 7; ++k) {  // union rows of pieces 0 (k 0,1), 1 (k 2,3), 2 (k 4,5,6)
        const int u = k < 2 ? lr + 64 * k : k < 4 ? 128 + lr + 64 * (k - 2) : 256 + lr + 64 * (k - 4);
        const int ip = u / C::S, q = u - ip * C::S;
        const int f = f0 - 1 + ip, p = p0 + q;
        const bool ok = u < C::UROWS && ip <= F + 1 && p < P;
        xo[k] = (ok && f >= 0 && f < T) ? (uint32_t)((bb * T + f) * P + p) * (uint32_t)D * 2u + 16u * lc : kOob;
        if (k == 0 && ok && f == -1) co = (uint32_t)(bb * P + p) * (uint32_t)D * 2u + 16u * lc;
    }
    const bool cache_rows = f0 == 0 && wave < 5;  // wave-uniform: union rows 0..39 of piece 0
    const int nkk = D / C::BK, KT = 3 * nkk;

    u32x4 rw[3], rx[3];
    auto load_w = [&](int t) {  // W slice of stage t = (chunk t / 3, offset t % 3)
        const int kk = t / 3, seg = t - 3 * kk;
        const uint32_t wk = (uint32_t)seg * (uint32_t)D * (uint32_t)D * 2u + (uint32_t)kk * (C::BK * 2);
        rw[0] = buf_load16(rW, wo[0] + wk);
        rw[1] = buf_load16(rW, wo[1] + wk);
        if (wave < 4) rw[2] = buf_load16(rW, wo[2] + wk);
    };
    auto load_x = [&](int kk, int piece) {  // piece of the union of chunk kk
        const uint32_t kb = (uint32_t)kk * (C::BK * 2);
        if (piece == 0) {
            rx[0] = buf_load16(rX, xo[0] + kb);
            if (cache_rows) rx[0] |= buf_load16(rC, co + kb);
            rx[1] = buf_load16(rX, xo[1] + kb);
        } else if (piece == 1) {
            rx[0] = buf_load16(rX, xo[2] + kb);
            rx[1] = buf_load16(rX, xo[3] + kb);
        } else {
            rx[0] = buf_load16(rX, xo[4] + kb);
            rx[1] = buf_load16(rX, xo[5] + kb);
            if (wave < 2) rx[2] = buf_load16(rX, xo[6] + kb);
        }
    };
    auto store_w = [&](int buf) {
        uint16_t* st = wbuf0 + buf * C::WSTAGE;
        *(u32x4*)(st + tc_off(lr, lc)) = rw[0];
        *(u32x4*)(st + tc_off(lr + 64, lc)) = rw[1];
        if (wave < 4) *(u32x4*)(st + tc_off(lr + 128, lc)) = rw[2];
    };
    auto store_x = [&](int buf, int piece) {
        uint16_t* st = xbuf0 + buf * C::XSTAGE;
        const int u0 = 128 * piece + lr;
        *(u32x4*)(st + tc_off(u0, lc)) = rx[0];
        *(u32x4*)(st + tc_off(u0 + 64, lc)) = rx[1];
        if (piece == 2 && wave < 2) *(u32x4*)(st + tc_off(u0 + 128, lc)) = rx[2];
    };

    // Compute role: wave (wn, wm) owns channels 80 wn .. +79 and tile rows
    // 80 wm .. +79.  Fragment lane layout (16 x 16 x 32): lane l reads row
    // l % 16 of a 16-row block at k chunk l / 16 (8 consecutive k).
    const int wn = wave & 1, wm = wave >> 1;
    const int fr = lane & 15, fc = lane >> 4;
    f32x4 acc[C::WN][C::WM];
#pragma unroll
    for (int i = 0; i < C::WN; ++i)
#pragma unroll
        for (int j = 0; j < C::WM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Pipeline.  Stage t = (chunk kk, offset seg) computes from W buffer t & 1
    // and union buffer kk & 1.  At its end it stores what the previous stage's
    // loads brought (W of stage t + 1, piece seg of the union of chunk kk + 1;
    // both buffers' readers passed the last barrier) and loads W of stage t + 2
    // and the next piece.
    load_w(0);
    store_w(0);
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        load_x(0, s);
        store_x(0, s);
    }
    if (KT > 1) load_w(1);
    if (nkk > 1) load_x(1, 0);
    lds_barrier();
    for (int kk = 0; kk < nkk; ++kk) {
#pragma unroll
        for (int seg = 0; seg < 3; ++seg) {  // unrolled: the union piece is a constant
            const int t = 3 * kk + seg;
            const uint16_t* wb = wbuf0 + (t & 1) * C::WSTAGE;
            const uint16_t* xb = xbuf0 + (kk & 1) * C::XSTAGE;
#pragma unroll
            for (int ks = 0; ks < C::BK / 32; ++ks) {
                bf16x8 xf[C::WM];
#pragma unroll
                for (int j = 0; j < C::WM; ++j)
                    xf[j] = *(const bf16x8*)(xb + tc_off(80 * wm + 16 * j + fr + C::S * seg, 4 * ks + fc));
#pragma unroll
                for (int i = 0; i < C::WN; ++i) {
                    const bf16x8 wf = *(const bf16x8*)(wb + tc_off(80 * wn + 16 * i + fr, 4 * ks + fc));
#pragma unroll
                    for (int j = 0; j < C::WM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[j], acc[i][j], 0, 0, 0);
                }
            }
            if (t + 1 < KT) store_w((t + 1) & 1);
            if (kk + 1 < nkk) store_x((kk + 1) & 1, seg);
            if (t + 2 < KT) load_w(t + 2);
            // the piece the next stage stores: piece seg + 1 of chunk kk + 1, or
            // piece 0 of chunk kk + 2
            if (seg < 2) {
                if (kk + 1 < nkk) load_x(kk + 1, seg + 1);
            } else {
                if (kk + 2 < nkk) load_x(kk + 2, 0);
            }
            lds_barrier();
        }
    }

    // Epilogue: lane holds C[n][m] for the token of tile row .. + lane % 16 and
    // channels n = .. + 4 (lane / 16) + (0..3): 4 consecutive channels of one token.
#pragma unroll
    for (int j = 0; j < C::WM; ++j) {
        const int r = 80 * wm + 16 * j + fr, i = r / C::S, q = r - i * C::S;
        const int f = f0 + i, p = p0 + q;
        if (i >= F || f >= T || p >= P) continue;
        const int m = (bb * T + f) * P + p;
#pragma unroll
        for (int i2 = 0; i2 < C::WN; ++i2) {
            const int n = n0 + 80 * wn + 16 * i2 + 4 * fc;
            if (n >= D) continue;
            const size_t o = (size_t)m * D + n;
            const uint2 xv = *(const uint2*)(a.X + o);
            float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (a.bias) bv = *(const float4*)(a.bias + n);
            const float y0 = bf_lo(xv.x) + acc[i2][j][0] + bv.x;
            const float y1 = bf_hi(xv.x) + acc[i2][j][1] + bv.y;
            const float y2 = bf_lo(xv.y) + acc[i2][j][2] + bv.z;
            const float y3 = bf_hi(xv.y) + acc[i2][j][3] + bv.w;
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
