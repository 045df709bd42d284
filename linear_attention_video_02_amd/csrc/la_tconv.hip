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

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 15] (expcnt and lgkmcnt
// left unconstrained): vector-memory operations of this wave may stay in
// flight, the oldest first to complete.  The LDS-DMA loads below are counted
// by vmcnt but not tracked by the compiler, so their completion is awaited here.
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
#define LA_VMCNT_CASE(k) case k: __builtin_amdgcn_s_waitcnt(0x0F70 | k); break;
        LA_VMCNT_CASE(0) LA_VMCNT_CASE(1) LA_VMCNT_CASE(2) LA_VMCNT_CASE(3)
        LA_VMCNT_CASE(4) LA_VMCNT_CASE(5) LA_VMCNT_CASE(6) LA_VMCNT_CASE(7)
        LA_VMCNT_CASE(8) LA_VMCNT_CASE(9) LA_VMCNT_CASE(10) LA_VMCNT_CASE(11)
        LA_VMCNT_CASE(12) LA_VMCNT_CASE(13) LA_VMCNT_CASE(14)
#undef LA_VMCNT_CASE
        default: __builtin_amdgcn_s_waitcnt(0x0F70 | 15); break;
    }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier without the memory model's fences.  A release fence on
// LDS would drain vmcnt (it counts the LDS-DMA loads as LDS stores in flight)
// and so every prefetch at each barrier.  Here LDS is written only by those
// loads, whose completion each wave awaits itself (wait_vmcnt) before the
// barrier, and every LDS read has returned before its value is used, ahead of
// the barrier.  The empty asm statements keep the compiler from moving memory
// operations across it.
__device__ __forceinline__ void dma_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One wave-wide LDS-DMA load: lane i reads 16 bytes at byte offset off of
// the buffer r and writes them to LDS at dst + 16 i (dst wave-uniform).
// Offsets past the buffer's range write zeros.
__device__ __forceinline__ void dma16(BufRsrc r, uint32_t off, uint16_t* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, off, 0, 0, 0);
}

// FULL: tiles of 8 frames x 40 positions (blocks of 8 frames or more), with
// the tile shape known at compile time; otherwise F and S come from the
// arguments.
template <bool FULL>
__global__ __launch_bounds__(TconvCfg::THREADS) void la_tconv_bf16_kernel(TconvArgs a) {
    using C = TconvCfg;
    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t* const wbuf0 = lds;                          // W slice of a stage, three buffers
    uint16_t* const xbuf0 = lds + 3 * C::WSTAGE;          // frame union of a chunk, two buffers

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
    // Token tile mt: frames f0 .. f0 + F - 1 by positions p0 .. p0 + S - 1 of
    // batch element bb (S = 40 for F = 8; more positions for shorter blocks, a
    // multiple of 8); tile row r = S i + q holds token (f0 + i, p0 + q).  Its
    // frame union, frames f0 - 1 .. f0 + F, is staged per 64-channel chunk as
    // union rows u = S i' + q (frame f0 - 1 + i'), so time offset o in {-1, 0, 1}
    // of tile row r is union row r + S (o + 1).
    const int F = FULL ? 8 : a.F, S = FULL ? 40 : a.S, D = a.D, P = a.P, T = a.T;
    const int pt = mt % a.npt, ft = (mt / a.npt) % a.nft, bb = mt / (a.npt * a.nft);
    const int f0 = ft * F, p0 = pt * S, n0 = nt * C::BN;

    // Loads go straight from memory into LDS (LDS DMA), 8 rows of 128 bytes
    // per wave instruction: lane i fills row 8 q + i / 8 at slot i % 8, which
    // under the swizzle holds chunk c = (i % 8) ^ (i / 8).  W slice: 20
    // instructions, q = wave + 8 j (3 per wave for waves 0-3, else 2).  Union:
    // 50, q = wave + 8 j (7 for waves 0-1, else 6).  kOob (past every buffer's
    // range) loads zeros: channels past D, positions past P, frames past the
    // block (its zero padding frame) and union rows past frame f0 + F.  Union
    // frame -1 (a block's first tiles, union rows 0 .. S - 1 = instructions
    // 0 .. S/8 - 1, whole instructions since S is a multiple of 8) comes from
    // the cache.
    constexpr uint32_t kOob = 0x80000000u;
    const BufRsrc rX = make_rsrc(a.X, (uint32_t)((size_t)a.M * D * 2));
    const BufRsrc rC = make_rsrc(a.cache, (uint32_t)((size_t)(a.M / (T * P)) * P * D * 2));
    const BufRsrc rW = make_rsrc(a.W, (uint32_t)((size_t)3 * D * D * 2));
    const uint32_t cb = 16u * (uint32_t)((lane & 7) ^ (lane >> 3));  // byte offset of this lane's chunk
    const int nw = wave < 4 ? 3 : 2, nx = wave < 2 ? 7 : 6;
    uint32_t wo[3], xo[7];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int row = 8 * (wave + 8 * j) + (lane >> 3), n = n0 + row;
        wo[j] = (j < nw && n < D) ? (uint32_t)n * (uint32_t)D * 2u + cb : kOob;
    }
    uint32_t cache_j = 0;  // bit j: instruction j of this wave loads union frame -1 (wave-uniform)
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        const int u = 8 * (wave + 8 * j) + (lane >> 3);
        const int ip = u / S, q = u - ip * S;
        const int f = f0 - 1 + ip, p = p0 + q;
        const bool ok = j < nx && ip <= F + 1 && p < P;
        const bool from_cache = f0 == 0 && 8 * (wave + 8 * j) < S;
        if (from_cache) cache_j |= 1u << j;
        if (from_cache)
            xo[j] = p < P ? (uint32_t)(bb * P + p) * (uint32_t)D * 2u + cb : kOob;
        else
            xo[j] = (ok && f >= 0 && f < T) ? (uint32_t)((bb * T + f) * P + p) * (uint32_t)D * 2u + cb : kOob;
    }
    const int nkk = D / C::BK, KT = 3 * nkk;
    auto dma_w = [&](int t, int buf) {  // W slice of stage t = (chunk t / 3, offset t % 3)
        const int kk = t / 3, seg = t - 3 * kk;
        const uint32_t wk = (uint32_t)seg * (uint32_t)D * (uint32_t)D * 2u + (uint32_t)kk * (C::BK * 2);
        uint16_t* dst = wbuf0 + buf * C::WSTAGE + 8 * 64 * wave;
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (j < nw) dma16(rW, wo[j] + wk, dst + j * 8 * 8 * 64);
    };
    auto dma_x = [&](int kk, int buf) {  // frame union of chunk kk
        const uint32_t kb = (uint32_t)kk * (C::BK * 2);
        uint16_t* dst = xbuf0 + buf * C::XSTAGE + 8 * 64 * wave;
#pragma unroll
        for (int j = 0; j < 7; ++j) {
            if (j >= nx) break;
            dma16((cache_j >> j) & 1u ? rC : rX, xo[j] + kb, dst + j * 8 * 8 * 64);
        }
    };

    // Compute role: wave (wn, wm) owns channels 80 wn .. +79 and tile rows
    // 80 wm .. +79.  Fragment lane layout (16 x 16 x 32): lane l reads row
    // l % 16 of a 16-row block at k chunk l / 16 (8 consecutive k).
    const int wn = wave & 1, wm = wave >> 1;
    const int fr = lane & 15, fc = lane >> 4;
    // First tile row of fragment j of this wave, for reads of the frame union.
    // A fragment holding a real token (tile row < F S) maps, shifted by up to
    // 2 S, to union rows below (F + 2) S <= 400 (also when F S is not a
    // multiple of 16).  In a short block (F S < 320) a fragment with no real
    // token reads rows of fragment 0 instead (wave-uniform choice; its
    // results are never stored), so no read leaves the buffer.
    const int fs = F * S;
    auto frow = [&](int j) { const int r0 = 80 * wm + 16 * j; return r0 < fs ? r0 : 0; };
    // Accumulators start at the bias (4 consecutive channels per lane); the
    // shortcut X is added from LDS at the stage that holds it (below).
    f32x4 acc[C::WN][C::WM];
#pragma unroll
    for (int i = 0; i < C::WN; ++i) {
        const int n = n0 + 80 * wn + 16 * i + 4 * fc;
        f32x4 b0 = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.bias && n < D) b0 = *(const f32x4*)(a.bias + n);
#pragma unroll
        for (int j = 0; j < C::WM; ++j) acc[i][j] = b0;
    }

    // Pipeline.  Stage t = (chunk kk, offset seg) computes from W buffer
    // t % 3 = seg and union buffer kk & 1.  At its start it issues the loads
    // of W for stage t + 2 (into buffer (t + 2) % 3, whose readers, stage
    // t - 1, passed the last barrier) and, at seg 0, of the union of chunk
    // kk + 1 (into buffer (kk + 1) & 1, free since chunk kk - 1 ended): two
    // and three stages ahead of their use.  Before its closing barrier each
    // wave waits for its own loads other than those just issued, which covers
    // everything stage t + 1 reads.
    //
    // Each stage's barrier sits between its two k steps: by then the wave has
    // issued all of the stage's fragment reads, so past the barrier it reads
    // the next stage's first-step fragments (into the registers the first
    // step's MFMAs just freed) while the second step's MFMAs run, and the
    // next stage starts with its operands in registers.
    // Every fragment's first row is a multiple of 16, so its swizzle is that
    // of row fr: tc_off(r0 + fr, c) = 64 r0 + tc_off(fr, c).  A lane keeps the
    // two k steps' offsets; the rest is wave-uniform.
    const int lx0 = tc_off(fr, fc), lx1 = tc_off(fr, 4 + fc);
    const int wrow = 64 * 80 * wn;
    // 25 MFMAs with 10 fragment reads spread evenly among them (one after
    // every two MFMAs): measured 1.6% faster than a read pair after every
    // five; reading earlier than this pushes the kernel past 256 registers.
#define LA_TC_SCHED_GROUPS()                                                                  \
    for (int g = 0; g < 10; ++g) {                                                            \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); /* MFMAs */                        \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); /* DS reads */                     \
    }                                                                                         \
    __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
    auto read_step = [&](bf16x8 (&xf)[C::WM], bf16x8 (&wf)[C::WN], const uint16_t* xs, const uint16_t* wb,
                         int ks) {
        const int lx = ks ? lx1 : lx0;
#pragma unroll
        for (int j = 0; j < C::WM; ++j) xf[j] = *(const bf16x8*)(xs + 64 * frow(j) + lx);
#pragma unroll
        for (int i = 0; i < C::WN; ++i) wf[i] = *(const bf16x8*)(wb + wrow + 64 * 16 * i + lx);
    };
    dma_x(0, 0);
    dma_w(0, 0);
    if (KT > 1) dma_w(1, 1);
    wait_vmcnt(KT > 1 ? nw : 0);
    dma_barrier();
    bf16x8 xf0[C::WM], wf0[C::WN];  // first k step of the coming stage
    read_step(xf0, wf0, xbuf0, wbuf0, 0);
    for (int kk = 0; kk < nkk; ++kk) {
#pragma unroll
        for (int seg = 0; seg < 3; ++seg) {  // unrolled: buffer indices are constants
            const int t = 3 * kk + seg;
            int issued = 0;
            if (seg == 0 && kk + 1 < nkk) {
                dma_x(kk + 1, (kk + 1) & 1);
                issued += nx;
            }
            if (t + 2 < KT) {
                dma_w(t + 2, (seg + 2) % 3);
                issued += nw;
            }
            const uint16_t* wb = wbuf0 + seg * C::WSTAGE;
            const uint16_t* xb = xbuf0 + (kk & 1) * C::XSTAGE;
            const uint16_t* xs = xb + S * seg * 64;  // union rows shifted by this offset (S % 8 == 0:
                                                     // the swizzle of row u + S seg is that of row u)
            static_assert(C::BK == 64, "two 32-deep k steps per stage");
            // first k step (fragments read before the stage) with the second
            // step's 10 reads, two after every five MFMAs
            bf16x8 xf1[C::WM], wf1[C::WN];
            read_step(xf1, wf1, xs, wb, 1);
#pragma unroll
            for (int i = 0; i < C::WN; ++i)
#pragma unroll
                for (int j = 0; j < C::WM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf0[i], xf0[j], acc[i][j], 0, 0, 0);
            LA_TC_SCHED_GROUPS();
            wait_vmcnt(issued);
            dma_barrier();
            // second k step with the next stage's first-step reads (after the
            // last stage these read stale LDS into registers nobody uses: no
            // condition, so that the reads and MFMAs share one block and can
            // be interleaved)
            {
                const int sn = seg == 2 ? 0 : seg + 1, kn = seg == 2 ? kk + 1 : kk;
                const uint16_t* xbn = xbuf0 + (kn & 1) * C::XSTAGE;
                read_step(xf0, wf0, xbn + S * sn * 64, wbuf0 + sn * C::WSTAGE, 0);
            }
#pragma unroll
            for (int i = 0; i < C::WN; ++i)
#pragma unroll
                for (int j = 0; j < C::WM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf1[i], xf1[j], acc[i][j], 0, 0, 0);
            LA_TC_SCHED_GROUPS();
            if (seg == 1) {
                // The shortcut: the union's own-frame rows of chunk kk hold X for the
                // 16-channel blocks of this wave that fall in the chunk (a block never
                // straddles two chunks).  Each lane adds its token's 4 channels.
#pragma unroll
                for (int i = 0; i < C::WN; ++i) {
                    const int nb = n0 + 80 * wn + 16 * i;  // wave-uniform
                    if ((nb >> 6) != kk) continue;
                    const int e = (nb & 63) + 4 * fc;      // element within the chunk's 64
#pragma unroll
                    for (int j = 0; j < C::WM; ++j) {
                        const uint2 xv =
                            *(const uint2*)(xb + S * 64 + tc_off(frow(j) + fr, e >> 3) + (e & 7));
                        acc[i][j] += f32x4{bf_lo(xv.x), bf_hi(xv.x), bf_lo(xv.y), bf_hi(xv.y)};
                    }
                }
            }
        }
    }

    // Epilogue.  Lane holds Y[m][n .. n + 3] (bias and shortcut already in)
    // for the token of tile row .. + lane % 16 and channels n = .. + 4 (lane /
    // 16).  The tile is rounded to bf16 into LDS (free now: every wave passed
    // the last barrier, and no load is in flight), rows of 168 elements so the
    // 16 rows of one write land in distinct banks, then written out as 16-byte
    // pieces, 20 per token row of 160 channels, so that every store
    // instruction moves whole row segments.
    constexpr int YROW = 168;
    uint16_t* const ys = lds;
#pragma unroll
    for (int j = 0; j < C::WM; ++j)
#pragma unroll
        for (int i2 = 0; i2 < C::WN; ++i2) {
            const f32x4 y = acc[i2][j];
            *(uint2*)(ys + (80 * wm + 16 * j + fr) * YROW + 80 * wn + 16 * i2 + 4 * fc) =
                make_uint2(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]));
        }
    lds_barrier();
    constexpr int PIECES = C::BM * (C::BN / 8);
#pragma unroll 4
    for (int c = tid; c < PIECES; c += C::THREADS) {
        const int r = c / (C::BN / 8), k = c - r * (C::BN / 8);
        const int i = r / S, q = r - i * S;
        const int f = f0 + i, p = p0 + q, n = n0 + 8 * k;
        if (i >= F || f >= T || p >= P || n >= D) continue;
        *(u32x4*)(a.Y + (size_t)((bb * T + f) * P + p) * D + n) = *(const u32x4*)(ys + r * YROW + 8 * k);
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
    // set on every call (a host-side attribute, cheap): it must hold on the
    // device current at this launch
    const bool full = a.F == 8 && a.S == 40;
    void (*k)(TconvArgs) = full ? la_tconv_bf16_kernel<true> : la_tconv_bf16_kernel<false>;
    const hipError_t e =
        hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, TconvCfg::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(a.mtiles * a.ntiles), dim3(TconvCfg::THREADS), TconvCfg::LDS_BYTES, st, a);
    return hipGetLastError();
}

hipError_t la_tconv_cache_launch(const TconvCacheArgs& c, hipStream_t st) {
    const size_t pieces = (size_t)c.B * c.P * c.D / 8;
    hipLaunchKernelGGL(la_tconv_cache_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st, c);
    return hipGetLastError();
}
