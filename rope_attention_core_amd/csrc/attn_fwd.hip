// Fused RoPE attention forward for gfx950 (MI355X): RoPE(Q), RoPE(K) in FP32 with a
// cast back to the IO dtype, S = scale * Q K^T on MFMA, an FP32 online softmax,
// O += P V on MFMA, an optional sliding window and a two-branch differential variant.
//
// The method is the attention core described in the "Fixes the medium DiT's
// FP16-mixed ONNX so the attention core runs FP16" discussion (sections "The bug"
// and "The fix": RoPE in FP32, cast back, then a fused FP16 core whose softmax
// accumulates in FP32) and in the Stable Audio 3 TensorRT engines README (sections
// "How the kernels differ" and "Building your own": differential sliding-window
// attention, window of +-WINDOW keys, FP32 subtraction).
//
// Work decomposition (one workgroup = 4 waves = one tile of BM query rows of one
// (b, h) slab; one wave = QB blocks of 32 query rows):
//
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{f16,bf16}:
//    A = K tile rows (keys) from LDS, B = the wave's rotated Q held in registers for
//    the whole kernel. In the 32x32 accumulator a lane owns ONE query (lane % 32) and
//    16 keys, so the row max and row sum are per-lane reductions plus one exchange
//    with lane ^ 32 (v_permlane32_swap).
//  * O^T = V^T P^T with v_mfma_f32_32x32x16_f16: B = P^T comes straight from the
//    softmax registers (the key order inside an MFMA step is permuted to match the
//    accumulator layout, and V^T is read with the same permutation), A = V^T is read
//    from a transposed V tile in LDS.
//  * K is rotated (FP32, fixed operation order, no contraction) and rounded to the
//    IO dtype while it is staged into LDS; Q once into registers. V is staged
//    transposed; for bf16 inputs it is converted to fp16 on the way, so P and V
//    meet in fp16 (P rounded to fp16 keeps 11 significant bits).
//  * LDS is double buffered: the global loads of tile t+1 are in flight while tile
//    t is multiplied; one barrier per tile.
//  * Softmax in base 2 (scale * log2 e folded into one FMA) with a lazy rescale: the
//    running maximum used as the exponent base is only raised when a tile's maximum
//    exceeds it by more than TAU, so P stays below 2^TAU and most tiles skip the
//    O *= alpha pass. The result is the same softmax (any common base cancels).
//  * Tiles wholly outside the window are never visited; tiles that meet the window
//    edge or the end of the sequence are masked element-wise.
//  * Workgroup ids are remapped so that the workgroups one XCD receives (the
//    hardware deals them round robin over the 8 XCDs) are consecutive tiles of the
//    same heads, keeping each head's K/V in one XCD's L2.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

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

constexpr int IO_F16 = 0;
constexpr int IO_BF16 = 1;
constexpr int OUT_F16 = 0;
constexpr int OUT_BF16 = 1;
constexpr int OUT_F32 = 2;

constexpr int HD = 64;           // head dim
constexpr int NPAIR = HD / 2;    // cos/sin row length
constexpr int BN = 64;           // keys per tile
constexpr int NT = 256;          // threads per workgroup
constexpr int KS_STRIDE = 72;    // LDS row stride of the K tile in 16-bit elements
constexpr int VT_STRIDE = 68;    // LDS row stride of the V^T tile in 16-bit elements
constexpr float TAU = 8.0f;      // lazy-rescale threshold in log2 units

struct Params {
    const uint16_t *q, *k, *v;
    const float *cos, *sin;
    void *out;
    long long branch_stride;     // elements from branch 1 to branch 2 of q / k
    int L, window, n_qtiles, out_dtype, neg_scale;
    float lam, c;                // c = |scale| * log2(e)
};

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

// Round two floats to nearest-even in the IO dtype and pack them (a in the low half).
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
__device__ __forceinline__ u32x4 rope8(u32x4 x, f32x4 c, f32x4 s) {
#pragma clang fp contract(off)
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float x0, x1;
        unpack2<IO>(x[j], x0, x1);
        const float a = x0 * c[j];
        const float b = x1 * s[j];
        const float e = x0 * s[j];
        const float f = x1 * c[j];
        r[j] = pack2<IO>(a - b, e + f);
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

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ f32x4 ld16f(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// One branch's running softmax state for one 32-query block.
struct RowState {
    f32x16 o[2];     // O^T accumulators for d blocks 0..31 and 32..63
    float m;         // exponent base in log2 units (-inf before any valid key)
    float l;         // this lane's partial sum of P (its 16 keys of each 32)
};

// Softmax of one 32-query block over one 64-key tile, S^T layout; rescales the
// state when needed and returns P^T packed as fp16 MFMA B operands [kb][tt].
template <bool MASK>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[2], RowState &st, u32x4 (&p)[2][2], float c,
                                             int k0, int qi, int L, int window, int g) {
    const float NEG_INF = -__builtin_inff();
    if constexpr (MASK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + kb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
                const int dist = key - qi;
                const bool ok = key < L && (window < 0 || (dist <= window && dist >= -window));
                s[kb][i] = ok ? s[kb][i] : NEG_INF;
            }
    }
    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = pair_max(mx);
    const float mt = (mx == NEG_INF) ? NEG_INF : mx * c;
    const bool need = mt > st.m + TAU;
    if (__builtin_amdgcn_ballot_w64(need)) {
        const float mn = need ? mt : st.m;
        const float alpha = need ? __builtin_amdgcn_exp2f(st.m - mn) : 1.0f;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) st.o[db][i] *= alpha;
        st.l *= alpha;
        st.m = mn;
    }
    const float nb = (st.m == NEG_INF) ? 0.0f : -st.m;
    float sum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        float e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float v = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, nb));
            if constexpr (MASK) v = (s[kb][i] == NEG_INF) ? 0.0f : v;
            e[i] = v;
            sum += v;
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = pack2<IO_F16>(e[8 * tt + 2 * j], e[8 * tt + 2 * j + 1]);
            p[kb][tt] = w;
        }
    }
    st.l += sum;
}

template <int IO, bool DIFF, int QB>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(Params P) {
    constexpr int BM = 4 * 32 * QB;
    constexpr int KS_ELEMS = BN * KS_STRIDE;
    constexpr int VT_ELEMS = HD * VT_STRIDE;
    constexpr int NK = DIFF ? 2 : 1;
    constexpr int BUF_ELEMS = NK * KS_ELEMS + VT_ELEMS;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BUF_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 31;
    const int g = lane >> 5;
    const int L = P.L;
    const int window = P.window;
    const float c = P.c;

    // XCD-aware remap of the workgroup id (see the file header).
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int per = nblk >> 3, rem = nblk & 7, xcd = bid & 7, idx = bid >> 3;
    const int lid = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int bh = lid / P.n_qtiles;
    const int qt = lid - bh * P.n_qtiles;

    const size_t head = (size_t)bh * (size_t)L * HD;
    const uint16_t *Qh = P.q + head;
    const uint16_t *Kh = P.k + head;
    const uint16_t *Vh = P.v + head;
    const uint16_t *Q2h = P.q + P.branch_stride + head;
    const uint16_t *K2h = P.k + P.branch_stride + head;

    const int q0 = qt * BM;
    const int qw = q0 + wave * 32 * QB;

    // ---- Q (and Q2): rotate once into registers, B-operand layout ----------------
    u32x4 qreg[QB][4];
    u32x4 q2reg[DIFF ? QB : 1][4];
    const uint32_t qsign = P.neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw + qb * 32 + r;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int d0 = 16 * ks + 8 * g;
            u32x4 x = {0, 0, 0, 0}, x2 = {0, 0, 0, 0};
            f32x4 cc = {0.f, 0.f, 0.f, 0.f}, ss = {0.f, 0.f, 0.f, 0.f};
            if (qi < L) {
                x = ld16(Qh + (size_t)qi * HD + d0);
                if constexpr (DIFF) x2 = ld16(Q2h + (size_t)qi * HD + d0);
                cc = ld16f(P.cos + (size_t)qi * NPAIR + d0 / 2);
                ss = ld16f(P.sin + (size_t)qi * NPAIR + d0 / 2);
            }
            qreg[qb][ks] = rope8<IO>(x, cc, ss) ^ qsign;
            if constexpr (DIFF) q2reg[qb][ks] = rope8<IO>(x2, cc, ss) ^ qsign;
        }
    }

    // ---- key range of this query tile ------------------------------------------
    const int q_last = min(L, q0 + BM) - 1;
    int k_lo = 0, k_hi = L;
    if (window >= 0) {
        k_lo = max(0, q0 - window);
        k_hi = min(L, q_last + window + 1);
    }
    const int t_begin = k_lo / BN;
    const int t_end = (k_hi + BN - 1) / BN;

    // ---- tile loaders ------------------------------------------------------------
    // K: 512 chunks of 8 elements; chunk ch -> key ch / 8, d0 = 8 * (ch % 8).
    // V: 256 pair-chunks; thread -> keys 2p, 2p+1 (p = tid % 32), d0 = 8 * (tid / 32).
    u32x4 kraw[2], k2raw[DIFF ? 2 : 1], vraw[2];
    f32x4 craw[2], sraw[2];
    const int vp = tid & 31;
    const int vd0 = (tid >> 5) * 8;

    auto issue_loads = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ch = tid + NT * i;
            const int kj = k0 + (ch >> 3);
            const int d0 = (ch & 7) * 8;
            if (kj < L) {
                kraw[i] = ld16(Kh + (size_t)kj * HD + d0);
                if constexpr (DIFF) k2raw[i] = ld16(K2h + (size_t)kj * HD + d0);
                craw[i] = ld16f(P.cos + (size_t)kj * NPAIR + d0 / 2);
                sraw[i] = ld16f(P.sin + (size_t)kj * NPAIR + d0 / 2);
            } else {
                kraw[i] = u32x4{0, 0, 0, 0};
                if constexpr (DIFF) k2raw[i] = u32x4{0, 0, 0, 0};
                craw[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                sraw[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        const int ka = k0 + 2 * vp;
        vraw[0] = (ka < L) ? ld16(Vh + (size_t)ka * HD + vd0) : u32x4{0, 0, 0, 0};
        vraw[1] = (ka + 1 < L) ? ld16(Vh + (size_t)(ka + 1) * HD + vd0) : u32x4{0, 0, 0, 0};
    };

    auto stage = [&](int buf) {
        uint16_t *Ks = smem + buf * BUF_ELEMS;
        uint16_t *Vt = Ks + NK * KS_ELEMS;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ch = tid + NT * i;
            const int key = ch >> 3;
            const int d0 = (ch & 7) * 8;
            *reinterpret_cast<u32x4 *>(Ks + key * KS_STRIDE + d0) = rope8<IO>(kraw[i], craw[i], sraw[i]);
            if constexpr (DIFF)
                *reinterpret_cast<u32x4 *>(Ks + KS_ELEMS + key * KS_STRIDE + d0) =
                    rope8<IO>(k2raw[i], craw[i], sraw[i]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t wa = vraw[0][j >> 1], wb = vraw[1][j >> 1];
            const int sh = (j & 1) * 16;
            uint32_t w;
            if constexpr (IO == IO_BF16) {
                const float fa = __uint_as_float(((wa >> sh) & 0xffffu) << 16);
                const float fb = __uint_as_float(((wb >> sh) & 0xffffu) << 16);
                w = pack2<IO_F16>(fa, fb);
            } else {
                w = ((wa >> sh) & 0xffffu) | (((wb >> sh) & 0xffffu) << 16);
            }
            *reinterpret_cast<uint32_t *>(Vt + (vd0 + j) * VT_STRIDE + 2 * vp) = w;
        }
    };

    // ---- running state -----------------------------------------------------------
    RowState st[QB], st2[DIFF ? QB : 1];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        st[qb].o[0] = f32x16{};
        st[qb].o[1] = f32x16{};
        st[qb].m = -__builtin_inff();
        st[qb].l = 0.0f;
        if constexpr (DIFF) {
            st2[qb].o[0] = f32x16{};
            st2[qb].o[1] = f32x16{};
            st2[qb].m = -__builtin_inff();
            st2[qb].l = 0.0f;
        }
    }

    const int qw_hi = qw + 32 * QB - 1;
    const bool wave_live = qw < L;

    issue_loads(t_begin);
    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        stage(buf);
        __syncthreads();
        if (t + 1 < t_end) issue_loads(t + 1);

        const int k0 = t * BN;
        bool skip = !wave_live;
        if (window >= 0) skip = skip || (k0 > qw_hi + window) || (k0 + BN - 1 < qw - window);
        if (skip) continue;
        const bool need_mask =
            (k0 + BN > L) || (window >= 0 && (k0 < qw_hi - window || k0 + BN - 1 > qw + window));

        const uint16_t *Ks = smem + buf * BUF_ELEMS;
        const uint16_t *Vt = Ks + NK * KS_ELEMS;

        // S^T = K Q^T for every query block; each K operand is read once per wave.
        f32x16 s[QB][2], s2[DIFF ? QB : 1][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            u32x4 ka[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) ka[ks] = ld16(Ks + (kb * 32 + r) * KS_STRIDE + 16 * ks + 8 * g);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma_qk<IO>(ka[ks], qreg[qb][ks], acc);
                s[qb][kb] = acc;
            }
            if constexpr (DIFF) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    ka[ks] = ld16(Ks + KS_ELEMS + (kb * 32 + r) * KS_STRIDE + 16 * ks + 8 * g);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    f32x16 acc = {};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) acc = mfma_qk<IO>(ka[ks], q2reg[qb][ks], acc);
                    s2[qb][kb] = acc;
                }
            }
        }

        // online softmax -> P^T in fp16
        u32x4 pp[QB][2][2], pp2[DIFF ? QB : 1][2][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int qi = qw + qb * 32 + r;
            if (need_mask) {
                softmax_tile<true>(s[qb], st[qb], pp[qb], c, k0, qi, L, window, g);
                if constexpr (DIFF) softmax_tile<true>(s2[qb], st2[qb], pp2[qb], c, k0, qi, L, window, g);
            } else {
                softmax_tile<false>(s[qb], st[qb], pp[qb], c, k0, qi, L, window, g);
                if constexpr (DIFF) softmax_tile<false>(s2[qb], st2[qb], pp2[qb], c, k0, qi, L, window, g);
            }
        }

        // O^T += V^T P^T; each V^T operand is read once per wave.
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const uint16_t *vrow = Vt + (db * 32 + r) * VT_STRIDE + kb * 32 + 16 * tt + 4 * g;
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow);
                    const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 8);
                    const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        st[qb].o[db] = mfma_pv(va, pp[qb][kb][tt], st[qb].o[db]);
                        if constexpr (DIFF) st2[qb].o[db] = mfma_pv(va, pp2[qb][kb][tt], st2[qb].o[db]);
                    }
                }
    }

    // ---- epilogue: normalise, subtract, cast, store rows < L ---------------------
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float inv = 1.0f / pair_sum(st[qb].l);
        float inv2 = 0.0f;
        if constexpr (DIFF) inv2 = 1.0f / pair_sum(st2[qb].l);
        const int qi = qw + qb * 32 + r;
        if (qi >= L) continue;
        const size_t row = head + (size_t)qi * HD;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o[j] = st[qb].o[db][grp * 4 + j] * inv;
                    if constexpr (DIFF) o[j] = o[j] - P.lam * (st2[qb].o[db][grp * 4 + j] * inv2);
                }
                const int d = db * 32 + grp * 8 + g * 4;
                if (P.out_dtype == OUT_F32) {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(P.out) + row + d) = f32x4{o[0], o[1], o[2], o[3]};
                } else if (P.out_dtype == OUT_BF16) {
                    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(P.out) + row + d) =
                        u32x2{pack2<IO_BF16>(o[0], o[1]), pack2<IO_BF16>(o[2], o[3])};
                } else {
                    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(P.out) + row + d) =
                        u32x2{pack2<IO_F16>(o[0], o[1]), pack2<IO_F16>(o[2], o[3])};
                }
            }
    }
}

template <int IO, bool DIFF, int QB>
hipError_t launch(const LaunchArgs &a, int n_qtiles) {
    Params P;
    P.q = static_cast<const uint16_t *>(a.q);
    P.k = static_cast<const uint16_t *>(a.k);
    P.v = static_cast<const uint16_t *>(a.v);
    P.cos = a.cos;
    P.sin = a.sin;
    P.out = a.out;
    P.branch_stride = (long long)a.B * a.H * a.L * HD;
    P.L = a.L;
    P.window = a.window;
    P.n_qtiles = n_qtiles;
    P.out_dtype = a.out_dtype;
    P.neg_scale = a.neg_scale;
    P.lam = a.lam;
    P.c = a.scale_log2;
    const unsigned grid = (unsigned)n_qtiles * (unsigned)a.B * (unsigned)a.H;
    hipLaunchKernelGGL((attn_fwd_kernel<IO, DIFF, QB>), dim3(grid), dim3(NT), 0,
                       static_cast<hipStream_t>(a.stream), P);
    return hipGetLastError();
}

// Query blocks of 32 rows per wave for an instance.
int pick_qb(const LaunchArgs &a) { return a.diff ? 1 : 2; }

}  // namespace

int tile_rows(const LaunchArgs &a) { return 4 * 32 * pick_qb(a); }

int launch_forward(const LaunchArgs &a) {
    const int bm = tile_rows(a);
    const int n_qtiles = (a.L + bm - 1) / bm;
    const bool bf = a.dtype == 1;
    hipError_t e;
    if (a.diff) {
        e = bf ? launch<IO_BF16, true, 1>(a, n_qtiles) : launch<IO_F16, true, 1>(a, n_qtiles);
    } else {
        e = bf ? launch<IO_BF16, false, 2>(a, n_qtiles) : launch<IO_F16, false, 2>(a, n_qtiles);
    }
    return (int)e;
}

}  // namespace sa3
