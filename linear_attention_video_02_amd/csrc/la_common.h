// Device helpers shared by the linear-attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ---------------------------------------------------------------------------
// exact division by a runtime constant: q = floor(n / d) for 0 <= n < 2^31
// (Granlund-Montgomery round-up multiplier: m = floor(2^(31+l) / d) + 1 with
//  l = ceil(log2 d); then m*d - 2^(31+l) <= d <= 2^l, which makes
//  floor(n*m / 2^(31+l)) exact for every n < 2^31, and n*m < 2^64.)
// ---------------------------------------------------------------------------
struct FastDiv {
    uint64_t m;
    uint32_t shift;  // 31 + l
    uint32_t d;
};

static inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    FastDiv f;
    f.shift = 31 + l;
    f.m = ((1ull << f.shift) / d) + 1;
    f.d = d;
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (uint32_t)(((uint64_t)n * f.m) >> f.shift);
}

// ---------------------------------------------------------------------------
// geometry of one call: tokens, grid and RoPE pair split
// ---------------------------------------------------------------------------
struct LaGeom {
    int BH;        // batch * heads
    int ntok;      // tokens per (batch, head) in the arrays of this call
    int n_offset;  // global index of the arrays' token 0 (block-causal mode)
    int rope;      // 0: no positional rotation
    int gh, gw;    // grid plane (gt only matters for validation)
    int pt, ph, pw;  // rotation pairs per axis
    FastDiv div_hw, div_w;
};

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_round(float a) {
    return bf_lo(pack_bf16(a, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// RoPE table in LDS.  Layout (float2 = (cos, sin)):
//   [0, nt*pt)            t rows  t_lo .. t_lo+nt-1, pt pairs each
//   [nt*pt, +gh*ph)       h rows  0 .. gh-1,          ph pairs each
//   [.., +gw*pw)          w rows  0 .. gw-1,          pw pairs each
// Angles: pos * 10000^(-k/P_a) evaluated in fp64, reduced to [-pi, pi] in
// fp64, then sin/cos in fp32 (|error| ~ 3e-7 for any position).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int rope_table_entries(int nt, const LaGeom& g) {
    return nt * g.pt + g.gh * g.ph + g.gw * g.pw;
}

__device__ inline void build_rope_table(float2* tab, int t_lo, int nt, const LaGeom& g) {
    const double kLog2Base = 13.287712379549449;      // log2(10000)
    const double kInv2Pi = 0.15915494309189535;
    const double k2PiHi = 6.283185307179586;
    const double k2PiLo = 2.4492935982947064e-16;
    const int nT = nt * g.pt, nH = g.gh * g.ph, nW = g.gw * g.pw;
    for (int i = threadIdx.x; i < nT + nH + nW; i += blockDim.x) {
        int pos, k, np;
        if (i < nT) {
            pos = t_lo + i / g.pt; k = i % g.pt; np = g.pt;
        } else if (i < nT + nH) {
            int j = i - nT; pos = j / g.ph; k = j % g.ph; np = g.ph;
        } else {
            int j = i - nT - nH; pos = j / g.pw; k = j % g.pw; np = g.pw;
        }
        double omega = exp2(-((double)k / (double)np) * kLog2Base);
        double ang = (double)pos * omega;
        double q = rint(ang * kInv2Pi);
        double r = fma(-q, k2PiHi, ang);
        r = fma(-q, k2PiLo, r);
        float s, c;
        sincosf((float)r, &s, &c);
        tab[i] = make_float2(c, s);
    }
}

// Where pair p's (cos, sin) lives: entry = base + pos_axis * stride.
struct PairRef {
    int base, stride, axis;
};

__device__ __forceinline__ PairRef pair_ref(int p, int nt, const LaGeom& g) {
    PairRef r;
    if (p < g.pt) {
        r.base = p; r.stride = g.pt; r.axis = 0;
    } else if (p < g.pt + g.ph) {
        r.base = nt * g.pt + (p - g.pt); r.stride = g.ph; r.axis = 1;
    } else {
        r.base = nt * g.pt + g.gh * g.ph + (p - g.pt - g.ph); r.stride = g.pw; r.axis = 2;
    }
    return r;
}

// (t - t_lo, h, w) of global token n
struct Pos3 {
    int t, h, w;
};

__device__ __forceinline__ Pos3 token_pos(uint32_t n, int t_lo, const LaGeom& g) {
    uint32_t t = fdiv(n, g.div_hw);
    uint32_t r = n - t * (uint32_t)(g.gh * g.gw);
    uint32_t h = fdiv(r, g.div_w);
    Pos3 p;
    p.t = (int)t - t_lo;
    p.h = (int)h;
    p.w = (int)(r - h * (uint32_t)g.gw);
    return p;
}

__device__ __forceinline__ int pair_entry(const PairRef& r, const Pos3& p) {
    int pos = r.axis == 0 ? p.t : (r.axis == 1 ? p.h : p.w);
    return r.base + pos * r.stride;
}

// rotate (x0, x1) by the angle whose (cos, sin) is cs
__device__ __forceinline__ void rotate(float& x0, float& x1, float2 cs) {
    float a = x0 * cs.x - x1 * cs.y;
    float b = x0 * cs.y + x1 * cs.x;
    x0 = a;
    x1 = b;
}
