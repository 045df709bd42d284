// Device helpers shared by the linear-attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ---------------------------------------------------------------------------
// exact division by a runtime constant: q = floor(n / d) for 0 <= n < 2^31.
// With l = ceil(log2 d) >= 1 and m = ceil(2^(31+l) / d) (which fits 32 bits
// because d > 2^(l-1)), m*d - 2^(31+l) <= d - 1, so floor(n*m / 2^(31+l)) is
// exact whenever n*(d-1) < 2^(31+l), i.e. for every n < 2^31.  On the device
// that is one v_mul_hi_u32 and one shift.  d = 1 is flagged separately.
// ---------------------------------------------------------------------------
struct FastDiv {
    uint32_t m;
    uint32_t shift;  // l - 1
    uint32_t one;    // d == 1
    uint32_t d;
};

static inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.one = d == 1;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    if (l == 0) l = 1;
    const uint64_t k = 1ull << (31 + l);
    f.m = (uint32_t)((k + d - 1) / d);
    f.shift = l - 1;
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return f.one ? n : (__umulhi(n, f.m) >> f.shift);
}

// Channels a kernel works on for head dim d: d itself for 32, 64 and 128;
// d = 112 runs as 128 with channels 112..127 held at zero on chip (HBM rows
// keep their 112 channels).
template <int D>
struct Pad {
    static constexpr int P = D == 112 ? 128 : D;
};

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
    FastDiv div_pt, div_ph, div_pw;  // by the pair counts (RoPE table build)
};

// ---------------------------------------------------------------------------
// buffer loads/stores through a resource descriptor bounded to a byte range:
// reads past the range return 0 and writes past it are dropped, in hardware,
// so the ragged end of a token chunk needs no branches (and the compiler can
// keep counting outstanding loads exactly instead of draining them).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t BufRsrc;

__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t nbytes) {
    // third descriptor word for gfx9-family raw (stride 0) buffers
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

// Streaming loads of the inputs (Q, K, V: read once per pass) carry the
// non-temporal hint (cache policy nt).  Same-process A/B on gfx950, outputs
// bitwise equal: 720p-5s state pass 61.4 -> 55.7 us, apply 62.5 -> 61.0 us;
// token-causal call 222 -> 220 us; N = 65,536 d = 128 step 420 -> 412 us.
// The scope bits (sc0, sc1) made no difference either way.
__device__ __forceinline__ u32x4 buf_load16(BufRsrc r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2v;
__device__ __forceinline__ u32x2v buf_load8(BufRsrc r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2);
}

__device__ __forceinline__ void buf_store16(u32x4 v, BufRsrc r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// Device-coherent load (cache policy sc1, device scope): served from the
// coherence point, never from a line another XCD's L2 may hold stale.  For
// data other workgroups of the same kernel wrote with device-scope stores.
__device__ __forceinline__ u32x4 buf_load16_dev(BufRsrc r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
}

// Device-coherent store (cache policy sc1): written through to the coherence
// point, for data that other workgroups of the same kernel read with
// buf_load16_dev once the store has completed.
__device__ __forceinline__ void buf_store16_dev(u32x4 v, BufRsrc r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 16);
}

// Streaming store for outputs nobody reads back soon (cache policy sc1 nt).
// A default store leaves the line dirty in the memory-side Infinity Cache; it
// is written to HBM later, while the next kernel streams its own inputs, and
// slows that kernel down (a K/V read kernel after a copy: 83 us with default
// stores, 47 us with these).  "nt" alone is pathological here: never use it
// without sc1.  Only for stores that cover whole 128-byte lines: partial lines
// written this way are not merged in L2 first (a d = 112 apply, whose rows
// straddle lines, ran 75% slower).
__device__ __forceinline__ void buf_store16_stream(u32x4 v, BufRsrc r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 16 | 2);
}

// Workgroup barrier for an LDS hand-off only.  __syncthreads() also orders
// global memory, which on gfx9 (loads and stores share vmcnt) drains every
// prefetched load before each barrier; this one waits for LDS operations only.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, output lane j,
// element e is element (j % 4) of what input lane 4e + j/4 addressed.  So if
// lane i of a group addresses X[r0 + i/4][c0 + 4*(i%4)] of a row-major bf16
// tile X[row][col], lane j receives X[r0 .. r0+3][c0 + j]: four consecutive
// rows of one column, which is half of an MFMA operand fragment whose k index
// runs along rows.  (Checked on the device with an in-bounds layout probe.)
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ s16x4 lds_read_tr4(const uint16_t* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(p));
}

// Two transposed reads -> one 8-element bf16 operand (rows r0..r0+7 of one column).
__device__ __forceinline__ bf16x8 lds_read_tr8(const uint16_t* p_rows0_3, const uint16_t* p_rows4_7) {
    const s16x4 a = lds_read_tr4(p_rows0_3);
    const s16x4 b = lds_read_tr4(p_rows4_7);
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, v);
}

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

// Split two floats into bf16 hi (truncated: the top 16 bits) and bf16 lo
// (x - hi, rounded to nearest even).  hi + lo equals x to 2^-16 relative.
// Returns (packed hi, packed lo).
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    hi = __builtin_amdgcn_perm(ub, ua, 0x07060302u);  // high halves: a in bits 0-15, b in 16-31
    lo = pack_bf16(a - __uint_as_float(ua & 0xffff0000u), b - __uint_as_float(ub & 0xffff0000u));
}

// two floats -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
    f16x2 v;
    v[0] = (_Float16)a;
    v[1] = (_Float16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Largest of the 8 bf16 values of a u32x4 as a non-negative 16-bit pattern:
// the signed 16-bit maximum of the raw words, clamped at 0 -- which is the
// largest relu'd value's bit pattern (non-negative bf16 values order like
// their int16 patterns; negative ones lie below 0).  The words are copied to
// scalars before the bit casts: this compiler turns __builtin_bit_cast of a
// vector-element expression (w[1]) into a cast of element 0.
typedef __attribute__((ext_vector_type(2))) short s16x2_t;
__device__ __forceinline__ s16x2_t as_s16x2(uint32_t x) { return __builtin_bit_cast(s16x2_t, x); }
__device__ __forceinline__ uint32_t max_relu_bits8(u32x4 w) {
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
    s16x2_t m = __builtin_elementwise_max(as_s16x2(w0), as_s16x2(w1));
    m = __builtin_elementwise_max(m, as_s16x2(w2));
    m = __builtin_elementwise_max(m, as_s16x2(w3));
    const int v = m[0] > m[1] ? m[0] : m[1];
    return v > 0 ? (uint32_t)v : 0u;
}

// wave-wide maximum of a float (every lane gets it)
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float bf16_round(float a) {
    return bf_lo(pack_bf16(a, 0.0f) & 0xffffu);
}

// relu of two packed bf16 values: a bf16 with the sign bit set reads as a
// negative int16 and a non-negative one as a non-negative int16, so a signed
// 16-bit max against 0 is relu (and maps -0 to +0).  One v_pk_max_i16.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
    typedef __attribute__((ext_vector_type(2))) short s16x2;
    s16x2 v = __builtin_bit_cast(s16x2, w);
    s16x2 z = {0, 0};
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(v, z));
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

// The table is followed in LDS by d/2 doubles of scratch (the frequencies),
// which the caller's LDS size must include.  Called by every thread of the
// workgroup; contains a workgroup barrier on LDS.
__device__ inline void build_rope_table(float2* tab, int t_lo, int nt, const LaGeom& g) {
    const double kLog2Base = 13.287712379549449;      // log2(10000)
    const double kInv2Pi = 0.15915494309189535;
    const double k2PiHi = 6.283185307179586;
    const double k2PiLo = 2.4492935982947064e-16;
    const int nT = nt * g.pt, nH = g.gh * g.ph, nW = g.gw * g.pw;
    // the frequency of each pair, once: pairs [0, pt) of axis t, then h, then w
    double* omg = (double*)(tab + nT + nH + nW);
    for (int i = threadIdx.x; i < g.pt + g.ph + g.pw; i += blockDim.x) {
        int k, np;
        if (i < g.pt) {
            k = i; np = g.pt;
        } else if (i < g.pt + g.ph) {
            k = i - g.pt; np = g.ph;
        } else {
            k = i - g.pt - g.ph; np = g.pw;
        }
        omg[i] = exp2(-((double)k / (double)np) * kLog2Base);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    for (int i = threadIdx.x; i < nT + nH + nW; i += blockDim.x) {
        int pos, j;  // position on the entry's axis, index of its frequency
        if (i < nT) {
            const int r = (int)fdiv((uint32_t)i, g.div_pt);
            pos = t_lo + r; j = i - r * g.pt;
        } else if (i < nT + nH) {
            const int r = i - nT;
            pos = (int)fdiv((uint32_t)r, g.div_ph); j = g.pt + r - pos * g.ph;
        } else {
            const int r = i - nT - nH;
            pos = (int)fdiv((uint32_t)r, g.div_pw); j = g.pt + g.ph + r - pos * g.pw;
        }
        double ang = (double)pos * omg[j];
        double q = rint(ang * kInv2Pi);
        double r = fma(-q, k2PiHi, ang);
        r = fma(-q, k2PiLo, r);
        float s, c;
        sincosf((float)r, &s, &c);
        tab[i] = make_float2(c, s);
    }
}

// Where pair p's (cos, sin) lives: entry = base + row offset of its axis,
// where the row offsets of a token are (t - t_lo) * pt, h * ph, w * pw.
// Packed in one register as base * 4 + axis.
typedef int PairRef;

__device__ __forceinline__ PairRef pair_ref(int p, int nt, const LaGeom& g) {
    if (p < g.pt) return p * 4;
    if (p < g.pt + g.ph) return (nt * g.pt + (p - g.pt)) * 4 + 1;
    return (nt * g.pt + g.gh * g.ph + (p - g.pt - g.ph)) * 4 + 2;
}

// Table row offsets of global token n: ((t - t_lo) * pt, h * ph, w * pw)
struct Pos3 {
    int t, h, w;
};

// All products here fit 24 bits (a grid whose RoPE table fits LDS has
// gh * gw < 2^24), so they use the full-rate 24-bit multiplier.
__device__ __forceinline__ Pos3 token_pos(uint32_t n, int t_lo, const LaGeom& g) {
    uint32_t t = fdiv(n, g.div_hw);
    uint32_t r = n - __umul24(t, (uint32_t)(g.gh * g.gw));
    uint32_t h = fdiv(r, g.div_w);
    Pos3 p;
    p.t = __mul24((int)t - t_lo, g.pt);
    p.h = __mul24((int)h, g.ph);
    p.w = __mul24((int)(r - __umul24(h, (uint32_t)g.gw)), g.pw);
    return p;
}

// Table entry of a pair for a token: base + the row offset of the pair's axis.
// Everything is passed by value and selected arithmetically: a select between
// fields of a struct held by reference gets turned into an indexed load from a
// private (scratch) array.
__device__ __forceinline__ int pair_entry(PairRef r, Pos3 p) {
    const int axis = r & 3;
    const int dh = axis >= 1 ? p.h - p.t : 0;
    const int dw = axis >= 2 ? p.w - p.h : 0;
    return (r >> 2) + p.t + dh + dw;
}

// Byte offsets of global token n's table rows: 8 (t - t_lo) pt, 8 h ph, 8 w pw
// (token_pos with the float2 entry size folded into the multipliers).
__device__ __forceinline__ Pos3 token_pos8(uint32_t n, int t_lo, const LaGeom& g) {
    uint32_t t = fdiv(n, g.div_hw);
    uint32_t r = n - __umul24(t, (uint32_t)(g.gh * g.gw));
    uint32_t h = fdiv(r, g.div_w);
    Pos3 p;
    p.t = __mul24((int)t - t_lo, 8 * g.pt);
    p.h = __mul24((int)h, 8 * g.ph);
    p.w = __mul24((int)(r - __umul24(h, (uint32_t)g.gw)), 8 * g.pw);
    return p;
}

// The table entries of four consecutive pairs p0 .. p0 + 3 (8 channels of
// one row, one lane).  Every axis has at least 3 pairs (P / 3 >= 3 from
// d = 18 on), so the four lie on at most two axes: A, pair 0's, and B, pair
// 3's.  For a token the lane forms the two row bases once,
//   ra = 8 (base of pair 0) + row offset of A,
//   rb = 8 (base of B's first pair k - k) + row offset of B,
// and pair i's entry is at byte (pair i on B ? rb : ra) + 8 i of the table:
// one select a pair, the + 8 i an immediate offset of the LDS read.
struct Rope4 {
    int xa, xb;            // 8 (base of pair 0), 8 (base of pair k - k)
    bool ah, aw, bh, bw;   // A / B is the h / the w axis
    bool onb1, onb2, onb3; // pair i (1..3) lies on B, B != A
};

__device__ __forceinline__ Rope4 rope4_make(int p0, int nt, const LaGeom& g) {
    auto axis = [&](int p) { return p < g.pt ? 0 : (p < g.pt + g.ph ? 1 : 2); };
    auto base = [&](int p) {
        const int a = axis(p);
        return a == 0 ? p : (a == 1 ? nt * g.pt + (p - g.pt) : nt * g.pt + g.gh * g.ph + (p - g.pt - g.ph));
    };
    const int A = axis(p0), B = axis(p0 + 3);
    int k = 3;
    while (k > 1 && axis(p0 + k - 1) == B) --k;  // first pair on B (k = 3 if only pair 3)
    Rope4 r;
    r.xa = 8 * base(p0);
    r.xb = A == B ? r.xa : 8 * (base(p0 + k) - k);
    r.ah = A == 1;
    r.aw = A == 2;
    r.bh = B == 1;
    r.bw = B == 2;
    r.onb1 = axis(p0 + 1) != A;
    r.onb2 = axis(p0 + 2) != A;
    r.onb3 = axis(p0 + 3) != A;
    return r;
}

// the two row bases of a token (p8 from token_pos8; passed by value: see
// pair_entry)
__device__ __forceinline__ int2 rope4_rows(Rope4 r, Pos3 p8) {
    const int oa = r.aw ? p8.w : (r.ah ? p8.h : p8.t);
    const int ob = r.bw ? p8.w : (r.bh ? p8.h : p8.t);
    return make_int2(oa + r.xa, ob + r.xb);
}

// rotate (x0, x1) by the angle whose (cos, sin) is cs
__device__ __forceinline__ void rotate(float& x0, float& x1, float2 cs) {
    float a = x0 * cs.x - x1 * cs.y;
    float b = x0 * cs.y + x1 * cs.x;
    x0 = a;
    x1 = b;
}

// rotate the four pairs of x by their entries of table tab (rows rr from
// rope4_rows); npairs = 2 rotates pairs 0 and 1 only
template <int NPAIRS = 4>
__device__ __forceinline__ void rope4_rotate(float (&x)[2 * NPAIRS], const float2* tab, Rope4 r, int2 rr) {
    const char* pa = (const char*)tab + rr.x;
    const char* pb = (const char*)tab + rr.y;
    rotate(x[0], x[1], *(const float2*)pa);
    rotate(x[2], x[3], *(const float2*)((r.onb1 ? pb : pa) + 8));
    if (NPAIRS > 2) {
        rotate(x[4 % (2 * NPAIRS)], x[5 % (2 * NPAIRS)], *(const float2*)((r.onb2 ? pb : pa) + 16));
        rotate(x[6 % (2 * NPAIRS)], x[7 % (2 * NPAIRS)], *(const float2*)((r.onb3 ? pb : pa) + 24));
    }
}
