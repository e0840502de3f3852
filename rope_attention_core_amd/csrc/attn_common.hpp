// Device-side building blocks shared by the gfx950 attention kernels: element
// conversions, the FP32 RoPE rotation, MFMA wrappers, lane-pair reductions, buffer
// loads, the tile mask and the softmax of one 32-query block. Included by each kernel
// source; everything lives in an anonymous namespace, one copy per translation unit.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "sa3attn_internal.hpp"

namespace sa3 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int IO_F16 = 0;
constexpr int IO_BF16 = 1;
constexpr int OUT_BF16 = 1;
constexpr int OUT_F32 = 2;

constexpr int HD = 64;            // head dim
constexpr int ROWB = HD * 2;      // bytes per q/k/v row, and per cos/sin row (32 floats)
constexpr int BN = 64;            // keys per tile
constexpr int NBUF = 3;           // LDS stages of the long-span kernel
constexpr int KS_STRIDE = 72;     // LDS row stride of the K tile in 16-bit elements
constexpr int VT_STRIDE = 72;     // LDS row stride of the V^T tile in 16-bit elements
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9)
constexpr float TAU = 8.0f;       // lazy rescale: a row's base moves only when its max passes it by more

struct Params {
    const uint16_t *q, *k, *v;
    const float *cos, *sin;
    void *out;
    long long q_br, k_br;         // elements from branch 1 to branch 2 of q / k
    long long qb, qh, kb, kh, vb, vh, ob, oh, ol;   // element strides of b and h (and l for out)
    uint32_t q_rowb, k_rowb, v_rowb;                // bytes from one position to the next
    int H, L, window, n_qtiles, out_dtype, neg_scale;
    float lam, c;                 // c = |scale| * log2(e)
    int rope_half, rot_dim;       // RoPE of the general instances: half-split pairs, rotary width
    uint32_t tab_rowb;            // bytes per cos/sin table row (rot_dim / 2 floats)
    // pre-pass workspace: K' [branch][B*H][Lp][D] rotated, in the IO type; V'
    // [B*H][Lp/64][D][64] fp16, each 64-key tile transposed (Lp = L rounded up to 64)
    uint16_t *kw, *vw;
    int ws_tiles;                 // Lp / 64
    int n_items;                  // query tiles x B x H (the long-span kernel's work items)
    int cp;                       // every item spans >= 3 key tiles (its pipeline may run on)
    // split tail (one-round-per-tile grids with the pre-pass): the last n_tail query tiles
    // are each split into n_split key ranges, one workgroup per range, after n_full whole
    // tiles; each range's (O, m, l) goes to `part`, and the workgroup that brings the
    // tile's counter in `cnt` to n_split merges them (n_split = 0: no split)
    int n_full, n_split, n_tail;
    float *part;
    uint32_t *cnt;
};

// Kernel parameters common to every instance (n_qtiles and window are set by the caller).
inline Params make_params(const LaunchArgs &a) {
    Params P;
    P.q = static_cast<const uint16_t *>(a.q);
    P.k = static_cast<const uint16_t *>(a.k);
    P.v = static_cast<const uint16_t *>(a.v);
    P.cos = a.cos;
    P.sin = a.sin;
    P.out = a.out;
    P.q_br = a.q_br;
    P.k_br = a.k_br;
    P.qb = a.qs[0];
    P.qh = a.qs[1];
    P.kb = a.ks[0];
    P.kh = a.ks[1];
    P.vb = a.vs[0];
    P.vh = a.vs[1];
    P.ob = a.os[0];
    P.oh = a.os[1];
    P.ol = a.os[2];
    P.q_rowb = (uint32_t)(a.qs[2] * 2);
    P.k_rowb = (uint32_t)(a.ks[2] * 2);
    P.v_rowb = (uint32_t)(a.vs[2] * 2);
    P.H = a.H;
    P.L = a.L;
    P.window = a.window;
    P.n_qtiles = 1;
    P.n_items = 0;
    P.cp = 0;
    P.out_dtype = a.out_dtype;
    P.neg_scale = a.neg_scale;
    P.lam = a.lam;
    P.c = a.scale_log2;
    P.rope_half = a.rope_half;
    P.rot_dim = a.rot_dim;
    P.tab_rowb = (uint32_t)(a.rot_dim / 2 * 4);
    const long long lp = ((long long)a.L + BN - 1) / BN * BN;
    P.ws_tiles = (int)(lp / BN);
    P.kw = a.prep ? static_cast<uint16_t *>(a.ws) : nullptr;
    P.vw = a.prep ? P.kw + (a.diff ? 2 : 1) * (long long)a.B * a.H * lp * a.D : nullptr;
    P.n_full = 0;
    P.n_split = 0;
    P.n_tail = 0;
    P.part = nullptr;
    P.cnt = nullptr;
    return P;
}

// The split tail's fields (tail_plan), for the long-span kernel and the pre-pass.
inline void set_tail(Params &P, const LaunchArgs &a) {
    const TailPlan t = tail_plan(a);
    if (t.k == 0) return;
    P.n_full = t.n_full;
    P.n_split = t.k;
    P.n_tail = t.n_tail;
    P.part = reinterpret_cast<float *>(static_cast<char *>(a.ws) + t.part_off);
    P.cnt = reinterpret_cast<uint32_t *>(static_cast<char *>(a.ws) + t.cnt_off);
}

// ---- element conversions -------------------------------------------------------

template <int IO>
__device__ __forceinline__ void unpack2(uint32_t u, float &a, float &b) {
    if constexpr (IO == IO_BF16) {
        a = __uint_as_float(u << 16);
        b = __uint_as_float(u & 0xffff0000u);
    } else {
        f16x2 h = __builtin_bit_cast(f16x2, u);
        a = (float)h[0];
        b = (float)h[1];
    }
}

// Round two floats to nearest-even in the given 16-bit type and pack them (a low).
template <int IO>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (IO == IO_BF16) {
        bf16x2 h = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, h);
    } else {
        f16x2 h = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, h);
    }
}

// RoPE on 8 consecutive elements (4 adjacent pairs) with their cos/sin, in FP32 with
// every product and sum rounded on its own, then rounded to the IO dtype.
template <int IO>
__device__ __forceinline__ u32x4 rope8(u32x4 x, u32x4 cw, u32x4 sw) {
#pragma clang fp contract(off)
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float x0, x1;
        unpack2<IO>(x[j], x0, x1);
        const float c = __uint_as_float(cw[j]);
        const float s = __uint_as_float(sw[j]);
        const float a = x0 * c;
        const float b = x1 * s;
        const float e = x0 * s;
        const float f = x1 * c;
        r[j] = pack2<IO>(a - b, e + f);
    }
    return r;
}

// ---- RoPE of the general instances --------------------------------------------
// Chunk c of a position (dims 8c .. 8c+7) under pairing `half` and rotary width R
// (a multiple of 16, <= D): mode 0 passes it through (c >= R/8); mode 1 rotates
// adjacent pairs with table floats 4c .. 4c+3; mode 2 (half-split, c < R/16) pairs
// it with chunk c + R/16 as the first members, mode 3 (R/16 <= c < R/8) with chunk
// c - R/16 as the second members, both with table floats 8j .. 8j+7 of j = c mod R/16.
struct RopeChunk {
    int mode;
    int partner;      // chunk index of the other pair members (modes 2 and 3)
    uint32_t toff;    // byte offset of the table floats inside a table row
};
__device__ __forceinline__ RopeChunk rope_chunk(int c, int half, int R) {
    RopeChunk k;
    const int h = R >> 4;     // chunks per half of the rotated dims
    if (c >= (R >> 3)) {
        k.mode = 0;
        k.partner = c;
        k.toff = 0;
    } else if (!half) {
        k.mode = 1;
        k.partner = c;
        k.toff = (uint32_t)c * 16;
    } else if (c < h) {
        k.mode = 2;
        k.partner = c + h;
        k.toff = (uint32_t)c * 32;
    } else {
        k.mode = 3;
        k.partner = c - h;
        k.toff = (uint32_t)(c - h) * 32;
    }
    return k;
}

// The rotation of one chunk in FP32, every product and sum rounded on its own, then
// RNE to the IO dtype. own / partner: the chunk and its partner chunk; c0, c1 / s0,
// s1: table floats 0-3 and 4-7 of the chunk's table slice (mode 1 uses c0 / s0).
template <int IO>
__device__ __forceinline__ u32x4 rope8_general(u32x4 own, u32x4 partner, u32x4 c0, u32x4 c1, u32x4 s0,
                                               u32x4 s1, int mode) {
#pragma clang fp contract(off)
    if (mode == 0) return own;
    if (mode == 1) return rope8<IO>(own, c0, s0);
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float o0, o1, p0, p1;
        unpack2<IO>(own[j], o0, o1);
        unpack2<IO>(partner[j], p0, p1);
        const float ca = __uint_as_float(j < 2 ? c0[2 * j] : c1[2 * j - 4]);
        const float cb = __uint_as_float(j < 2 ? c0[2 * j + 1] : c1[2 * j - 3]);
        const float sa = __uint_as_float(j < 2 ? s0[2 * j] : s1[2 * j - 4]);
        const float sb = __uint_as_float(j < 2 ? s0[2 * j + 1] : s1[2 * j - 3]);
        float ra, rb;
        if (mode == 2) {            // first members: x0 c - x1 s with x0 = own, x1 = partner
            ra = o0 * ca - p0 * sa;
            rb = o1 * cb - p1 * sb;
        } else {                    // second members: x0 s + x1 c with x0 = partner, x1 = own
            ra = p0 * sa + o0 * ca;
            rb = p1 * sb + o1 * cb;
        }
        r[j] = pack2<IO>(ra, rb);
    }
    return r;
}

template <int IO>
__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 acc) {
    if constexpr (IO == IO_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_pv(u32x4 a, u32x4 b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

// max / sum over the two lanes (l, l ^ 32) that hold the same query.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer over the L positions of one (b, h) slab whose rows are rowb bytes apart: the
// last row's 128 bytes end the range, so rows >= L (and negative rows, whose 32-bit
// offsets wrap far above it) read as zeros.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes);
__device__ __forceinline__ rsrc_t slab_rsrc(const uint16_t *base, long long elems, uint32_t rowb, int L,
                                            uint32_t rowbytes = ROWB) {
    return make_rsrc(base + elems, (uint32_t)(L - 1) * rowb + rowbytes);
}
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)RSRC_WORD3);
}
// 16- and 8-byte loads; bytes at or past num_records read as zero.
__device__ __forceinline__ u32x4 bload(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 bload8(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}

__device__ __forceinline__ u32x4 lds16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Validity of the keys of a masked tile for one lane: key offset o (0..63 inside the
// tile, as laid out in the S^T accumulator) is valid iff lo <= o - 4g <= lo + span,
// evaluated as one unsigned compare.
struct TileMask {
    int lo;           // first valid key offset relative to k0 + 4g
    uint32_t span;    // number of further valid offsets
};

// softmax of one 32-query block of one branch over one 64-key tile against the
// exponent base -nb: P^T packed as fp16 MFMA B operands [kb][tt].
template <bool MASK>
__device__ __forceinline__ void softmax_p(const f32x16 (&s)[2], float c, float nb, TileMask mk,
                                          u32x4 (&p)[2][2], float &rowsum) {
    const float NEG_INF = -__builtin_inff();
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        float e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float t = __builtin_fmaf(s[kb][i], c, nb);
            if constexpr (MASK) {
                const int o = kb * 32 + (i >> 2) * 8 + (i & 3);
                t = ((uint32_t)(o - mk.lo) <= mk.span) ? t : NEG_INF;
            }
            e[i] = __builtin_amdgcn_exp2f(t);
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f16x2 h = {(_Float16)e[8 * tt + 2 * j], (_Float16)e[8 * tt + 2 * j + 1]};
                w[j] = __builtin_bit_cast(uint32_t, h);
                // row sum of the rounded P (what the MFMA multiplies), four chains
                acc[2 * kb + tt] = __builtin_amdgcn_fdot2(h, f16x2{(_Float16)1.0f, (_Float16)1.0f},
                                                          acc[2 * kb + tt], false);
            }
            p[kb][tt] = w;
        }
    }
    rowsum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// softmax of one 32-query block over one 32-key half (kb) of a 64-key tile against the
// exponent base -nb: P^T packed as fp16 MFMA B operands [tt], and the FP32 sum of the
// rounded P (two chains).
template <bool MASK>
__device__ __forceinline__ void softmax_half(const f32x16 &s, int kb, float c, float nb, TileMask mk,
                                             u32x4 (&p)[2], float &rowsum) {
    const float NEG_INF = -__builtin_inff();
    float e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float t = __builtin_fmaf(s[i], c, nb);
        if constexpr (MASK) {
            const int o = kb * 32 + (i >> 2) * 8 + (i & 3);
            t = ((uint32_t)(o - mk.lo) <= mk.span) ? t : NEG_INF;
        }
        e[i] = __builtin_amdgcn_exp2f(t);
    }
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f16x2 h = {(_Float16)e[8 * tt + 2 * j], (_Float16)e[8 * tt + 2 * j + 1]};
            w[j] = __builtin_bit_cast(uint32_t, h);
            acc[tt] = __builtin_amdgcn_fdot2(h, f16x2{(_Float16)1.0f, (_Float16)1.0f}, acc[tt], false);
        }
        p[tt] = w;
    }
    rowsum = acc[0] + acc[1];
}

// ---- range guard of the bf16 -> fp16 V conversion -------------------------------
// P.V runs on fp16 operands for both IO types, and a bf16 V with |v| >= 65536 has no
// fp16 value (it would become inf). The kernels stage V unscaled; when an accumulator
// of a workgroup turns out non-finite they look up the largest finite |v| of the keys
// that workgroup visited and, if it lies beyond fp16's range, redo the work with V
// multiplied by 2^-shift while it is staged (exact: a power of two, the scaled values
// keep their 8 significant bits inside fp16's normal range) and the output multiplied
// by 2^shift. Finite inputs within fp16's range never take that path.

// Largest finite |x| among the 8 bf16 values of a 16-byte chunk, as its bit pattern
// without the sign (infinities and NaNs count as 0).
__device__ __forceinline__ uint32_t bf16_finite_absmax(u32x4 w) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = w[j] & 0x7fffu, hi = (w[j] >> 16) & 0x7fffu;
        m = max(m, lo < 0x7f80u ? lo : 0u);
        m = max(m, hi < 0x7f80u ? hi : 0u);
    }
    return m;
}

// The shift that brings the bf16 magnitude with bits `absbits` below 2^16: the values
// of its binade then scale to at most 65280, an fp16 value (0 when it already fits).
__device__ __forceinline__ int vshift_of(uint32_t absbits) {
    const int e = (int)(absbits >> 7);   // biased exponent
    return e >= 143 ? e - 142 : 0;
}

// 2^e as a float, -126 <= e <= 127.
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Whether p holds on any lane of the workgroup's NW waves (all threads call it; one
// barrier; `words` = NW words of LDS no other code uses between two calls).
template <int NW>
__device__ __forceinline__ bool wg_any(bool p, uint32_t *words) {
    const unsigned long long b = __ballot(p);
    if ((threadIdx.x & 63) == 0) words[threadIdx.x >> 6] = b != 0ull ? 1u : 0u;
    __syncthreads();
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) a |= words[i];
    return __builtin_amdgcn_readfirstlane(a) != 0;
}

// Maximum of x over the workgroup's NW waves (same rules as wg_any).
template <int NW>
__device__ __forceinline__ uint32_t wg_max(uint32_t x, uint32_t *words) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off, 64));
    if ((threadIdx.x & 63) == 0) words[threadIdx.x >> 6] = x;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) m = max(m, words[i]);
    return __builtin_amdgcn_readfirstlane(m);
}

// A sum of the accumulators that is finite exactly when all of them are (with V within
// fp16's range their sizes stay far below the float range: |O| <= 65504 l).
template <int N>
__device__ __forceinline__ bool acc_finite(const f32x16 (&o)[N], float l) {
    float s = l;
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += o[n][i];
    return __builtin_fabsf(s) <= 3.0e38f;
}

// max(a, b, c); the compiler emits one v_max3_f32 for it. MFMA results, selects between
// them and -inf count as canonical floats, so no quieting instructions are added; and,
// unlike inline assembly, the compiler sees the read of the MFMA result registers and
// inserts the wait states the hardware needs between an MFMA and a VALU read of its
// result (an inline-asm max that reads fresh MFMA results gets none and reads stale
// registers).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Maximum of 32 values as a tree of 3-input maxima (depth 3) rather than a chain.
__device__ __forceinline__ float max32(const float (&v)[32]) {
    float a[12];
#pragma unroll
    for (int i = 0; i < 10; ++i) a[i] = max3f(v[3 * i], v[3 * i + 1], v[3 * i + 2]);
    a[10] = v[30];
    a[11] = v[31];
    const float b0 = max3f(a[0], a[1], a[2]);
    const float b1 = max3f(a[3], a[4], a[5]);
    const float b2 = max3f(a[6], a[7], a[8]);
    const float b3 = max3f(a[9], a[10], a[11]);
    return max3f(max3f(b0, b1, b2), b3, b3);
}

// exact maximum of c * s over one 32-key half of a tile for this lane pair (log2 units)
__device__ __forceinline__ float half_max(const f32x16 &s, float c) {
    const float a0 = max3f(s[0], s[1], s[2]), a1 = max3f(s[3], s[4], s[5]), a2 = max3f(s[6], s[7], s[8]);
    const float a3 = max3f(s[9], s[10], s[11]), a4 = max3f(s[12], s[13], s[14]);
    return pair_max(max3f(max3f(a0, a1, a2), max3f(a3, a4, s[15]), a4)) * c;
}

// exact maximum of c * s over the valid keys of this lane pair (log2 units)
template <bool MASK>
// With MASK the masked scores are also written back as -inf, so the softmax that follows
// needs no mask of its own (c > 0: -inf * c + b = -inf, and 2^-inf = 0).
__device__ __forceinline__ float tile_max(f32x16 (&s)[2], float c, TileMask mk) {
    const float NEG_INF = -__builtin_inff();
    float v[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = s[kb][i];
            if constexpr (MASK) {
                const int o = kb * 32 + (i >> 2) * 8 + (i & 3);
                x = ((uint32_t)(o - mk.lo) <= mk.span) ? x : NEG_INF;
                s[kb][i] = x;
            }
            v[kb * 16 + i] = x;
        }
    const float mx = pair_max(max32(v));
    return (mx == NEG_INF) ? NEG_INF : mx * c;
}

}  // namespace
}  // namespace sa3
