// Key-split attention for grids that leave the chip under-filled, on gfx950: plain full
// attention at D = 64 on the pre-pass workspace (rotated K' and fp16 V^T tiles).
//
// The long-span kernel gives each wave 32 query rows and all their keys, so a call has
// only as many waves as 32-row blocks: B=1 H=24 L=1292 has 984, under one per SIMD of
// an MI355X (1024 SIMDs), and a SIMD needs two waves to overlap one wave's softmax with
// the other's MFMAs. Here a workgroup of 4 waves takes a tile of 64 query rows and
// splits its keys in two halves: waves 0 and 1 take the two 32-row blocks over the
// first half of the key tiles, waves 2 and 3 the same rows over the second half. Each
// wave runs the long-span kernel's online softmax over its half (the same arithmetic
// per element: S^T = K Q^T on MFMA, base-2 softmax with a lazy rescale, P rounded to
// fp16, O^T = V^T P^T on MFMA); at the end the second-half waves hand (O, m, l) to the
// first-half waves through LDS, which combine them as O = 2^(m0 - M) O0 + 2^(m1 - M) O1
// (l likewise, M the larger base) and store out = O / l. Two workgroups share a CU (73.7
// KB of LDS each), so every SIMD runs two waves. The sums over a row's keys are taken in
// a different order than in the long-span kernel, so the outputs differ from it in the
// last bits (both are held to the oracle).
//
// Key tiles are copied into LDS from the pre-pass workspace, one per half and step, into
// two buffers each for K and for V^T: step j stages K(j + 2) and V(j + 1) (loaded during
// step j - 1), loads K(j + 3) and V(j + 2), issues QK^T(j + 1) into a second score set,
// whose MFMAs run under the softmax of step j, then computes the softmax and P.V of
// step j; one barrier per step. The attention core is the one described in the "Fixes
// the medium DiT's FP16-mixed ONNX so the attention core runs FP16" discussion
// (sections "The bug" and "The fix").

#include "attn_common.hpp"

namespace sa3 {
namespace {

// SHARED: the grid has more workgroups than compute units, so two share a CU and each
// SIMD runs one wave of each. The SIMD issues for the older wave first; a wave then drops
// to the lower priority for the second half of each step, so the workgroup that is
// behind gets the issue slots until it reaches that point too. With one workgroup per CU
// the priority changes only cost time, and that instance keeps one priority.
template <int IO, bool SHARED>
__global__ __launch_bounds__(256, 2) void attn_split_kernel(Params P) {
    constexpr int NT = 256;
    constexpr int NW = 4;
    constexpr int D = 64;
    constexpr int RB = D * 2;
    constexpr int NKS = D / 16;                  // MFMA k-steps of QK^T
    constexpr int NDB = D / 32;                  // 32-wide d blocks of O
    constexpr int KSTR = D + 8;                  // LDS row stride of a K tile (16-bit elements)
    constexpr int KS_ELEMS = BN * KSTR;
    constexpr int VT_ELEMS = D * VT_STRIDE;
    constexpr int STAGE = 2 * (KS_ELEMS + VT_ELEMS);   // one buffer of K and of V^T per half
    constexpr int KC = BN * (D / 8) / NT;        // K' chunks (16 bytes) per thread per tile
    constexpr int VC = D * BN / (8 * NT);        // V' chunks per thread per tile
    constexpr int VD = BN * D / (2 * NT);        // d values per thread in the redo's V staging
    static_assert(KC == 2 && VC == 2 && VD == 8, "tile split");
    static_assert(2 * STAGE * 2 >= 2 * 34 * 64 * 4, "LDS too small for the merge");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
    __shared__ uint32_t guard[2 * NW];           // words of the V range guard's reductions

    const float NEG_INF = -__builtin_inff();
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qb = wave & 1;                     // query block of this wave
    const int kh = wave >> 1;                    // key half of this wave
    const int r = lane & 31;
    const int g = lane >> 5;
    const int L = P.L;
    const float c = P.c;

    // item -> (b*h, query tile of 64 rows), XCD-aware as in the long-span kernel
    const int n_items = P.n_items;
    const int it = blockIdx.x;
    const int per = n_items >> 3, rem = n_items & 7, xcd = it & 7, idx = it >> 3;
    const int lid = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int bh = lid / P.n_qtiles;
    const int qt = lid - bh * P.n_qtiles;
    const int qw = qt * 64 + qb * 32;
    const long long slab = (long long)bh * L * D;

    // key tiles: half 0 takes [0, T0), half 1 [T0, T); a step past T reads zeros (past
    // the workspace's range) and its keys, all >= L, are masked
    const int T = P.ws_tiles;
    const int T0 = (T + 1) >> 1;
    const long long lpd = (long long)T * BN * D;
    const rsrc_t rkw = make_rsrc(P.kw + (long long)bh * lpd, (uint32_t)lpd * 2);
    const rsrc_t rvw = make_rsrc(P.vw + (long long)bh * lpd, (uint32_t)lpd * 2);
    const rsrc_t rv = slab_rsrc(P.v, slab, RB, L, RB);      // input V (the guard's redo)
    const rsrc_t rq = slab_rsrc(P.q, slab, RB, L, RB);
    const rsrc_t rc = make_rsrc(P.cos, (uint32_t)L * RB);
    const rsrc_t rs = make_rsrc(P.sin, (uint32_t)L * RB);
    const uint32_t qsign = P.neg_scale ? 0x80008000u : 0u;

    // Q rotated into registers (MFMA B-operand layout)
    // The tile's 64 query rows are loaded once for the workgroup (both key halves use
    // them), two 16-byte chunks per thread with whole rows per wave load; they are
    // rotated into LDS (the first K buffer, before the first tile is staged there) once
    // the first tiles' loads are in flight, and each wave reads its B operands from there.
    constexpr int QS = KSTR;                     // LDS row stride of the rotated Q rows
    constexpr int QCH = 64 * (D / 8) / NT;       // Q chunks per thread
    static_assert(QCH == 2 && 64 * QS <= KS_ELEMS, "Q rows in one K buffer");
    u32x4 qreg[NKS], qraw[QCH], qcos[QCH], qsin[QCH];
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
        const int m = tid + NT * i;
        const uint32_t off = (uint32_t)(qt * 64 + m / 8) * RB + (uint32_t)(m % 8) * 16;
        qraw[i] = bload(rq, off);
        qcos[i] = bload(rc, off);
        qsin[i] = bload(rs, off);
    }

    // ---- staging: both halves' tiles of one step ------------------------------------
    // K tiles are staged two steps ahead of their use in P.V's step (QK^T(j + 1) runs in
    // step j), V tiles one step ahead; each has two LDS buffers per half.
    u32x4 rawk[2][KC], rawv[2][VC];
    float vsc = 1.0f;
    auto tile_of = [&](int h, int j) __attribute__((always_inline)) { return h ? T0 + j : j; };
    auto kbuf = [&](int slot, int h) __attribute__((always_inline)) { return smem + (slot * 2 + h) * KS_ELEMS; };
    auto vbuf = [&](int slot, int h) __attribute__((always_inline)) {
        return smem + 4 * KS_ELEMS + (slot * 2 + h) * VT_ELEMS;
    };
    auto load_k = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t t = (uint32_t)tile_of(h, j);
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                const int cc = tid + i * NT;
                rawk[h][i] = bload(rkw, (t * BN + (uint32_t)(cc >> 3)) * RB + (uint32_t)(cc & 7) * 16);
            }
        }
    };
    auto load_v = [&](int j, auto safe_tag) __attribute__((always_inline)) {
        constexpr bool SAFE = decltype(safe_tag)::value;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t t = (uint32_t)tile_of(h, j);
            if constexpr (SAFE) {
                // input V: keys 2p, 2p + 1 (p = tid % 32), VD values of d from VD * (tid / 32)
                const uint32_t off = (t * BN + 2 * (uint32_t)(tid & 31)) * RB + (uint32_t)(tid >> 5) * VD * 2;
                rawv[h][0] = bload(rv, off);
                rawv[h][1] = bload(rv, off + RB);
            } else {
#pragma unroll
                for (int i = 0; i < VC; ++i) rawv[h][i] = bload(rvw, t * (D * BN * 2) + (uint32_t)(tid + i * NT) * 16);
            }
        }
    };
    auto stage_k = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint16_t *Ks = kbuf(slot, h);
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                const int cc = tid + i * NT;
                *reinterpret_cast<u32x4 *>(Ks + (cc >> 3) * KSTR + (cc & 7) * 8) = rawk[h][i];
            }
        }
    };
    auto stage_v = [&](int slot, auto safe_tag) __attribute__((always_inline)) {
        constexpr bool SAFE = decltype(safe_tag)::value;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint16_t *Vt = vbuf(slot, h);
            if constexpr (SAFE) {
                // convert (scaled by vsc) and transpose: keys 2p, 2p + 1 at their P.V
                // operand positions (bits 2 and 3 of the key index swapped)
                const int k2 = 2 * (tid & 31);
                const int vpos = (k2 & ~12) | ((k2 & 4) << 1) | ((k2 & 8) >> 1);
                const int vd0 = (tid >> 5) * VD;
#pragma unroll
                for (int j = 0; j < VD; ++j) {
                    const uint32_t wa = rawv[h][0][j >> 1], wb = rawv[h][1][j >> 1];
                    uint32_t w;
                    if constexpr (IO == IO_BF16) {
                        const float fa = __uint_as_float((j & 1) ? (wa & 0xffff0000u) : (wa << 16)) * vsc;
                        const float fb = __uint_as_float((j & 1) ? (wb & 0xffff0000u) : (wb << 16)) * vsc;
                        w = pack2<IO_F16>(fa, fb);
                    } else {
                        w = (j & 1) ? __builtin_amdgcn_perm(wb, wa, 0x07060302u)
                                    : __builtin_amdgcn_perm(wb, wa, 0x05040100u);
                    }
                    *reinterpret_cast<uint32_t *>(Vt + (vd0 + j) * VT_STRIDE + vpos) = w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < VC; ++i) {
                    const int cv = tid + i * NT;
                    *reinterpret_cast<u32x4 *>(Vt + (cv >> 3) * VT_STRIDE + (cv & 7) * 8) = rawv[h][i];
                }
            }
        }
    };

    // S^T of this wave's 32 rows against key tile j of its half (K in buffer j & 1)
    auto qk = [&](int j, f32x16 (&s)[2]) __attribute__((always_inline)) {
        const uint16_t *Ks = kbuf(j & 1, kh);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            u32x4 ka[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) ka[ks] = lds16(Ks + (kb * 32 + r) * KSTR + 16 * ks + 8 * g);
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) acc = mfma_qk<IO>(ka[ks], qreg[ks], acc);
            s[kb] = acc;
        }
    };

    f32x16 o[NDB];
    float l = 0.0f, m = NEG_INF;

    // one step: stage K(j + 2) and V(j + 1), load K(j + 3) and V(j + 2), issue QK^T(j + 1)
    // into `nxt`, then the softmax and P.V of step j on `cur`. Past a half's last step the
    // tiles are the other half's or lie past the workspace (read as zeros): staged,
    // computed and never used, which keeps the step one block of straight-line code.
    const int steps = T0;
    auto step = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2], auto safe_tag) __attribute__((always_inline)) {
        if constexpr (SHARED) __builtin_amdgcn_s_setprio(1);
        stage_k(j & 1);
        stage_v((j + 1) & 1, safe_tag);
        load_k(j + 3);
        load_v(j + 2, safe_tag);
        qk(j + 1, nxt);
        const uint16_t *Vt = vbuf(j & 1, kh);
        const int k0 = tile_of(kh, j) * BN;
        auto softmax = [&](auto mask_tag) __attribute__((always_inline)) {
            constexpr bool MASK = decltype(mask_tag)::value;
            TileMask mk{0, 0};
            if constexpr (MASK) {
                const int lo = -(k0 + 4 * g), hi = L - 1 - (k0 + 4 * g);
                mk = hi < lo ? TileMask{1 << 20, 0u} : TileMask{lo, (uint32_t)(hi - lo)};
            }
            const float mt = tile_max<MASK>(cur, c, mk);
            const float mn = (mt > m + TAU) ? mt : m;
            const float ea = __builtin_amdgcn_exp2f(m - mn);
            const float a = (mn == m) ? 1.0f : ea;
            const bool moved = mn != m;
            m = mn;
            const float nb = (mn == NEG_INF) ? 0.0f : -mn;
            // O changes only where a row's base moved (elsewhere the factor is exactly 1)
            if (__builtin_expect(__any(moved), 0)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[db][i] *= a;
            }
            float part[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (SHARED && kb == 1) __builtin_amdgcn_s_setprio(0);
                u32x4 p[2];
                softmax_half<false>(cur[kb], kb, c, nb, mk, p, part[kb]);   // masked by tile_max
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        o[db] = mfma_pv(lds16(Vt + (db * 32 + r) * VT_STRIDE + kb * 32 + 16 * tt + 8 * g), p[tt],
                                        o[db]);
            }
            l = __builtin_fmaf(l, a, part[0] + part[1]);
        };
        if (k0 + BN > L)
            softmax(std::true_type{});
        else
            softmax(std::false_type{});
        __syncthreads();
    };

    // one pass over this wave's key half; SAFE: the V range guard's redo
    auto run = [&](auto safe_tag) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
        l = 0.0f;
        m = NEG_INF;
        load_k(0);
        load_v(0, safe_tag);
        if constexpr (!decltype(safe_tag)::value) {
#pragma unroll
            for (int i = 0; i < QCH; ++i) {
                const int m = tid + NT * i;
                *reinterpret_cast<u32x4 *>(smem + (m / 8) * QS + (m % 8) * 8) = rope8<IO>(qraw[i], qcos[i], qsin[i]) ^ qsign;
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qreg[ks] = lds16(smem + (qb * 32 + r) * QS + 16 * ks + 8 * g);
            __syncthreads();   // every wave has its Q before K(0) is staged over it
        }
        stage_k(0);
        stage_v(0, safe_tag);
        load_k(1);
        stage_k(1);
        __syncthreads();
        f32x16 sa[2], sb[2];
        qk(0, sa);
        load_k(2);
        load_v(1, safe_tag);
        __syncthreads();   // every wave has read K(0) before step 0 stages K(2) over it
        for (int j = 0; j < steps; j += 2) {
            step(j, sa, sb, safe_tag);
            if (j + 1 < steps) step(j + 1, sb, sa, safe_tag);
        }
    };
    run(std::false_type{});

    // ---- range guard of the bf16 -> fp16 V conversion (see attn_common.hpp) -------------
    int vshift = 0;
    if constexpr (IO == IO_BF16) {
        if (__builtin_expect(wg_any<NW>(!acc_finite(o, l), guard), 0)) {
            uint32_t mx = 0;
            for (int cc = tid; cc < L * (D / 8); cc += NT)
                mx = max(mx, bf16_finite_absmax(bload(rv, (uint32_t)(cc >> 3) * RB + (uint32_t)(cc & 7) * 16)));
            vshift = vshift_of(wg_max<NW>(mx, guard + NW));
            if (vshift > 0) {
                vsc = exp2i(-vshift);
                run(std::true_type{});
            }
        }
    }

    // ---- merge the halves, normalise, store rows < L -------------------------------------
    // The second-half waves hand O, m and l to the first-half waves of the same rows: element
    // e of lane x of query block qb at word (qb * 34 + e) * 64 + x (m at e = 32, l at 33).
    float *xb = reinterpret_cast<float *>(smem);
    __syncthreads();   // every wave is done with the staged tiles
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) xb[(qb * 34 + db * 16 + i) * 64 + lane] = o[db][i];
        xb[(qb * 34 + 32) * 64 + lane] = m;
        xb[(qb * 34 + 33) * 64 + lane] = l;
    }
    __syncthreads();
    if (kh == 1) return;
    const int qi = qw + r;
    if (qi >= L) return;
    {
        const float m1 = xb[(qb * 34 + 32) * 64 + lane];
        const float mx = fmaxf(m, m1);
        // a half with no valid key has m = -inf and contributes nothing (2^-inf = 0)
        const float a0 = __builtin_amdgcn_exp2f(m - mx);
        const float a1 = __builtin_amdgcn_exp2f(m1 - mx);
        l = a0 * l + a1 * xb[(qb * 34 + 33) * 64 + lane];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = a0 * o[db][i] + a1 * xb[(qb * 34 + db * 16 + i) * 64 + lane];
    }
    // (2^vshift undoes the guard's scaling of V; l >= 1, so inv * 2^vshift stays finite)
    const float inv = (1.0f / pair_sum(l)) * exp2i(vshift);
    const long long row = slab + (long long)qi * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = o[db][grp * 4 + j] * inv;
            const int d = db * 32 + grp * 8 + g * 4;
            if (P.out_dtype == OUT_F32) {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(P.out) + row + d) = f32x4{y[0], y[1], y[2], y[3]};
            } else if (P.out_dtype == OUT_BF16) {
                *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(P.out) + row + d) =
                    u32x2{pack2<IO_BF16>(y[0], y[1]), pack2<IO_BF16>(y[2], y[3])};
            } else {
                *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(P.out) + row + d) =
                    u32x2{pack2<IO_F16>(y[0], y[1]), pack2<IO_F16>(y[2], y[3])};
            }
        }
}

}  // namespace

// Plain full attention at D = 64, contiguous, default RoPE, with the pre-pass workspace.
bool split_applies(const LaunchArgs &a) {
    return a.D == 64 && !a.diff && a.contig && a.window < 0 && a.prep;
}

int launch_split(const LaunchArgs &a, int n_qtiles) {
    Params P = make_params(a);
    P.n_qtiles = n_qtiles;
    P.n_items = n_qtiles * a.B * a.H;
    const dim3 grid((unsigned)P.n_items), block(256);
    hipStream_t s = static_cast<hipStream_t>(a.stream);
    const bool shared = P.n_items > (a.n_cu > 0 ? a.n_cu : 256);
    if (a.dtype == 1) {
        if (shared)
            hipLaunchKernelGGL((attn_split_kernel<IO_BF16, true>), grid, block, 0, s, P);
        else
            hipLaunchKernelGGL((attn_split_kernel<IO_BF16, false>), grid, block, 0, s, P);
    } else {
        if (shared)
            hipLaunchKernelGGL((attn_split_kernel<IO_F16, true>), grid, block, 0, s, P);
        else
            hipLaunchKernelGGL((attn_split_kernel<IO_F16, false>), grid, block, 0, s, P);
    }
    return (int)hipGetLastError();
}

}  // namespace sa3
