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
// Work decomposition: one workgroup = 8 waves = one tile of query rows of one (b, h)
// slab (256 rows; 128 in the differential variant, where a pair of waves shares 32
// rows, one wave per softmax branch); one wave = 32 query rows of one branch; keys in
// tiles of 64.
//
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{f16,bf16}:
//    A = K tile rows (keys) from LDS, B = the wave's rotated Q, held in registers for
//    the whole kernel. In the 32x32 accumulator a lane owns ONE query (lane % 32) and
//    16 keys of each 32, so row statistics are per-lane plus one exchange with
//    lane ^ 32 (v_permlane32_swap).
//  * O^T = V^T P^T with v_mfma_f32_32x32x16_f16: B = P^T comes straight from the
//    softmax registers (the key order inside an MFMA step is permuted to match the
//    accumulator layout); A = V^T from a transposed V tile in LDS whose key positions
//    carry the same permutation, so each lane's operand is one 16-byte LDS read (the
//    8-byte reads run at half the LDS bandwidth). For bf16 inputs V is converted to
//    fp16 as it is staged, so P (rounded to fp16, 11 significant bits) and V meet in
//    fp16.
//  * K is rotated (FP32, fixed operation order, no contraction) and rounded to the IO
//    dtype while it is staged into LDS; Q once into registers.
//  * Instances of one round per query tile on the pre-pass workspace (all but the
//    differential D = 128 ones) walk the keys in pairs of tiles (128 keys per step, one barrier per pair; plain calls also
//    take one maximum, base move and O rescale per pair), with K and V^T in LDS rings
//    of four tiles each; see pair_block. The others:
//  * Software pipeline over key tiles with three LDS buffers and one barrier per tile.
//    The block for tile t first issues QK^T(t+1) into the second score set, so those
//    MFMAs run under the softmax of tile t (VALU); P.V(t) follows each 32-key half of
//    that softmax; then tile t+2 is rotated/transposed into LDS while the global loads
//    of tile t+3 are in flight.
//  * Online softmax in base 2 (scale * log2 e folded into one FMA) with a lazy
//    rescale: each row keeps an exponent base m; a tile moves it only when the tile's
//    maximum exceeds m by more than TAU (and on the row's first valid keys, where m is
//    set to the exact maximum). So P = 2^(s*c - m) <= 2^TAU fits fp16; O and the
//    running sum are multiplied on every tile by 2^(m_old - m_new), which is exactly 1
//    except on those rare tiles (a branch around the product made the register
//    allocator copy the 32 accumulator registers every tile). Any common base cancels
//    in O / l, so the result is the same softmax. Differential calls at D = 64 skip
//    the maximum on unmasked tiles: P is computed against the current base and the
//    half tile is redone with its exact maximum only when some P overflowed fp16.
//  * Out-of-range rows read as zeros through buffer loads (the hardware returns 0
//    past num_records), so tails need no branches; scores of keys >= L and outside
//    the window are set to -inf in the tiles that need a mask.
//  * Workgroup ids are remapped so that the workgroups one XCD receives (dealt round
//    robin over the 8 XCDs) are consecutive tiles of the same heads, keeping each
//    head's K/V in one XCD's L2.
//  * Grids of more query tiles than compute units with short key spans (a sliding
//    window) run persistent: one workgroup per compute unit takes several query tiles
//    in turn, and the key-tile pipeline runs on from one into the next (the last blocks
//    of a tile stage the next tile's first key tiles), so a tile's start (its first
//    loads and stages) no longer stalls the workgroup.
//  * One-round grids with the pre-pass whose last round would leave at least half the
//    compute units idle split the tiles of that round into key ranges, merged by the
//    range that finishes last (the split tail; see tail_plan).

#include <algorithm>

#include "attn_common.hpp"

namespace sa3 {
namespace {

template <int NDB>
struct Branch {
    f32x16 o[NDB];   // O^T accumulators for d in [32 db, 32 db + 32)
    float l;         // this lane's partial FP32 sum of P (its 16 keys of each 32)
    float m;         // exponent base in log2 units (-inf: no valid key yet)
    float a;         // factor taking O and l from the previous base to m
};

// Waves per workgroup: 8, two per SIMD, so that one wave's VALU work can issue while the
// other waits (a single wave issues a VALU op at best every ~5 cycles, half the SIMD's
// rate); registers <= 256 per wave.
template <int D>
constexpr int waves_for() { return 8; }

// Plain: each wave owns 32 query rows, BM = 32 x waves. Differential: wave w < waves/2
// takes the first softmax branch (Q1, K1) of query block w, wave waves/2 + w the second
// (Q2, K2) of block waves/2 - 1 - w; both branches of a block multiply the same staged
// V tile, BM = 16 x waves, and the second hands O2 / l2 to the first through LDS at the
// end. (Waves w and waves/2 + w share a SIMD; the reversed order pairs a block at one
// end of the tile with one at the other, so in a window's edge tiles, which lie wholly
// outside one of the two blocks' windows, one wave of the SIMD has no softmax to do.)
// CONTIG: q, k, v and out are contiguous [B][H][L][D] (q, k stacked [2][...]) with the
// default RoPE; the row strides are then compile-time constants, which keeps scalar
// registers free. D: head dim, 64 or 128. PRE: K and V come from the pre-pass
// workspace (attn_prep.hip), already rotated / converted and in the LDS layout, so
// staging a tile is a copy (CONTIG then concerns only q, out and the table of q).
// PERS: persistent grid (each workgroup takes several query tiles in turn, see the file
// header); the one-round instances (false) take one query tile per workgroup.
// NW: waves per workgroup (8; 2 for the 64-row tiles of under-filled grids, see
// small_grid below); the 8-wave instances keep <= 256 registers (two waves per SIMD),
// the 2-wave ones may use more (two of them share a CU, one wave per SIMD).
template <int IO, bool DIFF, bool CONTIG, int D, bool PRE, bool PERS, int NW = waves_for<D>(), bool TAIL = false>
__global__ __launch_bounds__(NW * 64, NW >= 4 ? 2 : 1) void attn_fwd_kernel(Params P) {
    static_assert(!TAIL || (!PERS && PRE && NW == waves_for<D>()), "the split tail is for one-round pre-pass grids");
    constexpr int NT = NW * 64;
    constexpr int NBS = DIFF ? 2 : 1;        // K tiles staged per key tile (one per branch)
    constexpr int WPB = NW / NBS;            // waves (32-row query blocks) per branch
    constexpr int BM = WPB * 32;
    constexpr int RB = D * 2;                // bytes per q/k/v row, and per default cos/sin row
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int KC = BN * CPR / NT;        // K chunks per thread per branch
    constexpr int NKS = D / 16;              // MFMA k-steps of QK^T
    constexpr int NDB = D / 32;              // 32-wide d blocks of O
    constexpr int KSTR = D + 8;              // LDS row stride of the K tile (16-bit elements)
    constexpr int VD = BN * D / (2 * NT);    // d values per thread in the V^T staging (2 keys each)
    static_assert((D == 64 || D == 128) && KC >= 1 && (VD == 4 || VD % 8 == 0), "head dim 64 or 128");
    using vraw_t = std::conditional_t<VD >= 8, u32x4, u32x2>;
    constexpr int NV = VD >= 8 ? VD / 8 : 1;     // V loads per key of a thread
    constexpr int KS_ELEMS = BN * KSTR;
    constexpr int VT_ELEMS = D * VT_STRIDE;
    constexpr int BUF_ELEMS = NBS * KS_ELEMS + VT_ELEMS;
    // CP: the staging pipeline runs on from one query tile of the workgroup into the next
    // (its first two key tiles are staged, and the third loaded, during the last blocks of
    // the previous one), so the O2 exchange of a differential epilogue needs LDS of its
    // own; there is no room for it at D = 128, where each query tile starts cold.
    constexpr bool CP = PERS && !(DIFF && D == 128);
    constexpr int XB_ELEMS = (CP && DIFF) ? WPB * 32 * D * 2 : 0;
    static_assert(!DIFF || CP || NBUF * BUF_ELEMS * 2 >= WPB * 32 * D * 4, "LDS too small for the O2 exchange");
    // PAIR: one-round instances with the pre-pass walk the keys 128 at a time (see
    // pair_block below), with rings of PR K tiles (each branch) and PR V^T tiles in LDS
    // (not differential D = 128: its rings would take 213 KB)
    constexpr bool PAIR = PRE && (D == 64 || !DIFF) && !PERS && NW == waves_for<D>();
    constexpr int PR = 4;
    constexpr int PAIR_ELEMS = PR * NBS * KS_ELEMS + PR * VT_ELEMS;
    constexpr int STAGE_ELEMS = (PAIR && PAIR_ELEMS > NBUF * BUF_ELEMS) ? PAIR_ELEMS : NBUF * BUF_ELEMS;
    __shared__ __attribute__((aligned(16))) uint16_t smem[STAGE_ELEMS + XB_ELEMS];
    __shared__ uint32_t guard[2 * NW];       // words of the V range guard's reductions

    const float NEG_INF = -__builtin_inff();
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wbr = DIFF ? wave / WPB : 0;   // this wave's softmax branch
    const int wq = DIFF ? (wbr ? WPB - 1 - wave % WPB : wave % WPB) : wave;   // this wave's query block
    const int r = lane & 31;
    const int g = lane >> 5;
    const int L = P.L;
    const int window = P.window;
    const float c = P.c;

    // Work items: the query tiles of every (b, h), n_items in all. The grid holds at most
    // one workgroup per compute unit and each takes items blockIdx.x, blockIdx.x +
    // gridDim.x, ... (gridDim.x is then a multiple of 8, so they share the XCD).
    const int n_items = P.n_items;
    const int nbh = n_items / P.n_qtiles;
    const uint32_t qrb = CONTIG ? (uint32_t)RB : P.q_rowb;
    const uint32_t krb = (CONTIG || PRE) ? (uint32_t)RB : P.k_rowb;
    const uint32_t vrb = CONTIG ? (uint32_t)RB : P.v_rowb;
    // contiguous stacked branches are B*H*L*D elements apart
    const long long qbr = CONTIG ? (long long)nbh * L * D : P.q_br;
    const long long kbr = CONTIG ? qbr : P.k_br;
    // cos/sin: [L][R/2] floats (R = D in the contiguous instances: 2 D bytes per row)
    const uint32_t trb = CONTIG ? (uint32_t)RB : P.tab_rowb;
    const rsrc_t rc = make_rsrc(P.cos, (uint32_t)L * trb);
    const rsrc_t rs = make_rsrc(P.sin, (uint32_t)L * trb);
    const int rhalf = P.rope_half, rdim = P.rot_dim;
    constexpr uint32_t NOWHERE = 0xfffffff0u;   // an offset past every buffer: reads zeros
    const uint32_t qsign = P.neg_scale ? 0x80008000u : 0u;

    // item -> (b*h, query tile, key-tile range), with the XCD-aware remap of the file
    // header (consecutive items of one XCD are consecutive tiles of the same heads)
    struct Item {
        int bh, qt, tb, te;
    };
    // the XCD-aware remap of workgroup (or item) `it` of n
    auto remap = [](int it, int n) __attribute__((always_inline)) {
        const int per = n >> 3, rem = n & 7, xcd = it & 7, idx = it >> 3;
        return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    };
    // linear tile id -> (b*h, query tile, key-tile range)
    auto tile_of_lid = [&](int lid) __attribute__((always_inline)) {
        Item x;
        if (PERS && DIFF && window >= 0) {
            // persistent differential windows: heads in groups of four, query tiles major
            // within a group, so that the workgroups an XCD runs at once share the cos/sin
            // rows of their spans (and a head's neighbouring spans) while the group's K1,
            // K2 and V still fit its L2: 98 against 132 MB fetched per call at w = 256
            constexpr int G = 4;
            const int nq = P.n_qtiles, full = nbh / G;
            const int gl = G * nq;
            const int g = lid / gl;
            const int gs = g < full ? G : nbh - full * G;
            const int rr = lid - g * gl;
            x.qt = rr / gs;
            x.bh = g * G + (rr - x.qt * gs);
        } else {
            x.bh = lid / P.n_qtiles;
            x.qt = lid - x.bh * P.n_qtiles;
        }
        const int q0 = x.qt * BM;
        const int q_last = min(L, q0 + BM) - 1;
        int k_lo = 0, k_hi = L;
        if (window >= 0) {
            k_lo = max(0, q0 - window);
            k_hi = min(L, q_last + window + 1);
        }
        x.tb = k_lo / BN;
        x.te = (k_hi + BN - 1) / BN;
        return x;
    };
    auto item_at = [&](int it) __attribute__((always_inline)) { return tile_of_lid(remap(it, n_items)); };
    // K (each branch) and V of one (b, h): the pre-pass workspace or the inputs
    auto kv_of = [&](int bh, rsrc_t (&kk)[NBS], rsrc_t &vv) __attribute__((always_inline)) {
        if constexpr (PRE) {
            // K' [branch][B*H][Lp][D] and V' [B*H][Lp/64][D][64]: Lp * 2D bytes per slab
            const long long lpd = (long long)P.ws_tiles * BN * D;
#pragma unroll
            for (int br = 0; br < NBS; ++br) kk[br] = make_rsrc(P.kw + ((long long)br * nbh + bh) * lpd, (uint32_t)lpd * 2);
            vv = make_rsrc(P.vw + (long long)bh * lpd, (uint32_t)lpd * 2);
        } else {
            const int bb = bh / P.H, hh = bh - bb * P.H;
            const long long slab = (long long)bh * L * D;
#pragma unroll
            for (int br = 0; br < NBS; ++br)
                kk[br] = slab_rsrc(P.k, br * kbr + (CONTIG ? slab : bb * P.kb + hh * P.kh), krb, L, RB);
            vv = slab_rsrc(P.v, CONTIG ? slab : bb * P.vb + hh * P.vh, vrb, L, RB);
        }
    };

    int item = blockIdx.x;
    Item cur = item_at(item);
    // split tail (one-round instances): workgroups from n_full on take key range `part`
    // of split tile `spl` (the tiles after the n_full whole ones), XCD-aware like the rest
    int spl = -1, part = 0;
    if constexpr (TAIL) {
        if (P.n_split > 0) {
            if (item < P.n_full) {
                cur = tile_of_lid(remap(item, P.n_full));
            } else {
                const int ls = remap(item - P.n_full, P.n_tail * P.n_split);
                spl = ls / P.n_split;
                part = ls - spl * P.n_split;
                cur = tile_of_lid(P.n_full + spl);
                const int tb = cur.tb, nt = cur.te - cur.tb;
                cur.tb = tb + nt * part / P.n_split;
                cur.te = tb + nt * (part + 1) / P.n_split;
            }
        }
    }
    rsrc_t rk[NBS], rv;
    kv_of(cur.bh, rk, rv);
    // the next item (persistent grids only)
    bool has_nxt = false;
    Item nxt = cur;
    rsrc_t nk[NBS], nv;
    if constexpr (PERS) {
        has_nxt = item + (int)gridDim.x < n_items;
        if (has_nxt) nxt = item_at(item + (int)gridDim.x);
        kv_of(nxt.bh, nk, nv);
    }

    // the input V rows of the current item (the range guard's redo reads them even when
    // the staging copies V' from the pre-pass workspace)
    rsrc_t rvr = rv;
    auto raw_v_of = [&](int bh) __attribute__((always_inline)) {
        if constexpr (PRE) {
            const int bb = bh / P.H, hh = bh - bb * P.H;
            return slab_rsrc(P.v, CONTIG ? (long long)bh * L * D : bb * P.vb + hh * P.vh, vrb, L, RB);
        } else {
            return rv;
        }
    };

    // per-item values the lambdas below read (set at the start of every item)
    int qw = 0, qhi_live = 0;
    u32x4 qreg[NKS];

    // ---- staging: global -> registers -> (rotate / transpose) -> LDS -------------
    // K (each branch): 64 rows x CPR chunks of 8 elements; chunk item i of a thread is
    // row (tid / CPR) + i * NT / CPR, dims 8 (tid % CPR) .. +7.
    // V: thread -> keys 2p, 2p+1 (p = tid % 32) and VD values of d from VD * (tid / 32).
    u32x4 rawk[NBS][KC], rawc[KC], raws[KC];
    u32x4 rawp[NBS][KC], rawc1[KC], raws1[KC];   // general instances: partner chunks, table floats 4-7
    vraw_t rawv[2][NV];
    constexpr int VC = D * BN / (8 * NT);     // 16-byte V' chunks per thread (pre-pass layout)
    u32x4 rawvp[VC];

    // per-lane parts of the staging offsets (one multiply each, here); the per-tile part
    // (k0 + i * NT / CPR) * row bytes is wave-uniform and comes from the scalar unit
    const RopeChunk kch = rope_chunk(tid % CPR, rhalf, rdim);
    const uint32_t kl = (uint32_t)(tid / CPR) * krb + (uint32_t)(tid % CPR) * 16;
    const uint32_t kpl = (uint32_t)(tid / CPR) * krb + (uint32_t)kch.partner * 16;
    const uint32_t cl = CONTIG ? (uint32_t)(tid / CPR) * RB + (uint32_t)(tid % CPR) * 16
                               : (uint32_t)(tid / CPR) * trb + kch.toff;
    // V staging: thread -> keys 2p, 2p+1 (p = tid % 32) and VD values of d from
    // VD * (tid / 32); computed once for the fused instances, and where used in the
    // pre-pass instances (whose fast path copies V' tiles and needs them only in the
    // guard's redo), so that those keep no registers for them
    const int vp_ = tid & 31;
    const int vd0_ = (tid >> 5) * VD;
    const int vpos_ = (2 * vp_ & ~12) | ((2 * vp_ & 4) << 1) | ((2 * vp_ & 8) >> 1);
    const uint32_t vl_ = (uint32_t)(2 * vp_) * vrb + (uint32_t)vd0_ * 2;
    auto v_lane = [&](int &vd0, int &vpos, uint32_t &vl) __attribute__((always_inline)) {
        if constexpr (PRE) {
            const int vp = tid & 31;
            vd0 = (tid >> 5) * VD;
            vpos = (2 * vp & ~12) | ((2 * vp & 4) << 1) | ((2 * vp & 8) >> 1);
            vl = (uint32_t)(2 * vp) * vrb + (uint32_t)vd0 * 2;
        } else {
            vd0 = vd0_;
            vpos = vpos_;
            vl = vl_;
        }
    };
    // SAFE (the redo of the V range guard, bf16 only): V comes from the input rows even
    // in the pre-pass instances and is scaled by vsc = 2^-shift as it is converted.
    auto load_raw = [&](const rsrc_t (&kk)[NBS], const rsrc_t &vv, int t, auto safe_tag) __attribute__((always_inline)) {
        constexpr bool VPRE = PRE && !decltype(safe_tag)::value;
        if constexpr (PRE) {
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                const uint32_t k0 = (uint32_t)(t * BN + i * (NT / CPR));
#pragma unroll
                for (int br = 0; br < NBS; ++br) rawk[br][i] = bload(kk[br], kl + k0 * RB);
            }
        } else {
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                const uint32_t k0 = (uint32_t)(t * BN + i * (NT / CPR));
#pragma unroll
                for (int br = 0; br < NBS; ++br) rawk[br][i] = bload(kk[br], kl + k0 * krb);
                if constexpr (CONTIG) {
                    rawc[i] = bload(rc, cl + k0 * RB);
                    raws[i] = bload(rs, cl + k0 * RB);
                } else {
                    const uint32_t to = kch.mode ? cl + k0 * trb : NOWHERE;
                    const uint32_t t1 = kch.mode >= 2 ? to + 16 : NOWHERE;
                    const uint32_t po = kch.mode >= 2 ? kpl + k0 * krb : NOWHERE;
#pragma unroll
                    for (int br = 0; br < NBS; ++br) rawp[br][i] = bload(kk[br], po);
                    rawc[i] = bload(rc, to);
                    raws[i] = bload(rs, to);
                    rawc1[i] = bload(rc, t1);
                    raws1[i] = bload(rs, t1);
                }
            }
        }
        if constexpr (VPRE) {
            // tiles past the last one lie past the buffer's range and read zeros
#pragma unroll
            for (int j = 0; j < VC; ++j) rawvp[j] = bload(vv, (uint32_t)t * (D * BN * 2) + (uint32_t)(tid + j * NT) * 16);
        } else {
            int vd0, vpos;
            uint32_t vl;
            v_lane(vd0, vpos, vl);
            const uint32_t k0 = (uint32_t)(t * BN);
            if constexpr (VD >= 8) {
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    rawv[0][n] = bload(vv, vl + k0 * vrb + 16 * n);
                    rawv[1][n] = bload(vv, vl + k0 * vrb + vrb + 16 * n);
                }
            } else {
                rawv[0][0] = bload8(vv, vl + k0 * vrb);
                rawv[1][0] = bload8(vv, vl + k0 * vrb + vrb);
            }
        }
    };

    // V^T key positions: bits 2 and 3 of the key index swapped, so that the 8 keys one
    // lane multiplies in a P.V step (see load_v_operands) are contiguous.
    const int kat = (tid / CPR) * KSTR + (tid % CPR) * 8;
    float vsc = 1.0f;   // 2^-shift of the V range guard's redo (SAFE staging only)
    auto stage = [&](int buf, auto safe_tag) __attribute__((always_inline)) {
        constexpr bool SAFE = decltype(safe_tag)::value;
        constexpr bool VPRE = PRE && !SAFE;
        uint16_t *Ks = smem + buf * BUF_ELEMS;
        uint16_t *Vt = Ks + NBS * KS_ELEMS;
#pragma unroll
        for (int i = 0; i < KC; ++i)
#pragma unroll
            for (int br = 0; br < NBS; ++br) {
                u32x4 rot;
                if constexpr (PRE)
                    rot = rawk[br][i];
                else if constexpr (CONTIG)
                    rot = rope8<IO>(rawk[br][i], rawc[i], raws[i]);
                else
                    rot = rope8_general<IO>(rawk[br][i], rawp[br][i], rawc[i], rawc1[i], raws[i], raws1[i], kch.mode);
                *reinterpret_cast<u32x4 *>(Ks + br * KS_ELEMS + kat + i * (NT / CPR) * KSTR) = rot;
            }
        if constexpr (VPRE) {
#pragma unroll
            for (int j = 0; j < VC; ++j) {
                const int cv = tid + j * NT;
                *reinterpret_cast<u32x4 *>(Vt + (cv >> 3) * VT_STRIDE + (cv & 7) * 8) = rawvp[j];
            }
            return;
        }
        int vd0, vpos;
        uint32_t vl;
        v_lane(vd0, vpos, vl);
#pragma unroll
        for (int j = 0; j < VD; ++j) {
            const uint32_t wa = rawv[0][j >> 3][(j >> 1) & 3], wb = rawv[1][j >> 3][(j >> 1) & 3];
            uint32_t w;
            if constexpr (IO == IO_BF16) {
                float fa = __uint_as_float((j & 1) ? (wa & 0xffff0000u) : (wa << 16));
                float fb = __uint_as_float((j & 1) ? (wb & 0xffff0000u) : (wb << 16));
                if constexpr (SAFE) {
                    fa *= vsc;
                    fb *= vsc;
                }
                w = pack2<IO_F16>(fa, fb);
            } else {
                w = (j & 1) ? __builtin_amdgcn_perm(wb, wa, 0x07060302u) : __builtin_amdgcn_perm(wb, wa, 0x05040100u);
            }
            *reinterpret_cast<uint32_t *>(Vt + (vd0 + j) * VT_STRIDE + vpos) = w;
        }
    };

    // ---- MFMA stages -----------------------------------------------------------
    // S^T = K Q^T for this wave's branch: [kb] = keys 32 kb .. 32 kb + 31 of the tile
    auto qk = [&](int buf, f32x16 (&s)[2]) __attribute__((always_inline)) {
        const uint16_t *Ks = smem + buf * BUF_ELEMS + wbr * KS_ELEMS;
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

    Branch<NDB> st;

    // mask of tile t for this wave's rows (lane-level lo/span)
    auto tile_mask = [&](int t, int kend) __attribute__((always_inline)) {
        const int k0 = t * BN;
        const int qi = qw + r;
        int lo = 0, hi = kend - 1;
        if (window >= 0 && qi < L) {
            lo = max(lo, qi - window);
            hi = min(hi, qi + window);
        }
        TileMask mk;
        lo -= k0 + 4 * g;
        hi -= k0 + 4 * g;
        if (hi < lo) {
            mk.lo = 1 << 20;
            mk.span = 0;
        } else {
            mk.lo = lo;
            mk.span = (uint32_t)(hi - lo);
        }
        return mk;
    };
    // the wave-uniform decision whether tile t needs element masks
    auto tile_needs_mask = [&](int t, int kend) __attribute__((always_inline)) {
        const int k0 = t * BN;
        if (k0 + BN > kend) return true;
        if (window < 0 || qw > qhi_live) return false;
        return k0 < qhi_live - window || k0 + BN - 1 > qw + window;
    };
    // a tile of the item's span that lies wholly outside this wave's window (its rows sit
    // at one end of the query tile): every score masked, so P = 0 and the base, O and l
    // stay as they are; the wave skips that tile's softmax and P.V (wave-uniform; the QK^T
    // issued for it a block earlier stays, a branch around it made the compiler spill).
    // Contiguous D = 64 instances only: in the others the branch adds spills.
    constexpr bool SKIP_OUT = D == 64 && CONTIG;
    auto tile_outside = [&](int t) __attribute__((always_inline)) {
        const int k0 = t * BN;
        return SKIP_OUT && window >= 0 && qw <= qhi_live && (k0 > qhi_live + window || k0 + BN - 1 < qw - window);
    };

    // Two score sets: the block of tile t starts QK^T(t+1) into sb[P^1] so its MFMAs run
    // under the softmax of tile t (sb[P]); P.V(t) follows each 32-key half of the softmax.
    // Staging t+2 and loading t+3 go first in the block (EARLY: the buffer of t+2 was
    // last read in tile t-1, which the barrier closed), so that the loads have a whole
    // tile to arrive before the next block's staging waits for them; placed after the
    // softmax, the compiler's register reuse makes the softmax wait for them instead.
    // The general fused instances keep them last: early, they spill.
    constexpr bool EARLY = PRE || CONTIG;
    // D = 128 doubles O and the rotated Q; two score sets would not fit in 256 registers,
    // so it computes QK^T(t) at the start of block t and relies on the other wave of its
    // SIMD to fill the wait for the MFMA results.
    constexpr bool PIPE2 = D == 64;
    // The overflow-checked softmax of unmasked tiles (below): 1-3% faster on
    // differential calls, 2.6% slower on plain ones (whose tile of 256 rows already keeps
    // the VALU busier per barrier), so differential D = 64 only.
    constexpr bool FAST = DIFF && D == 64;
    f32x16 sb[PIPE2 ? 2 : 1][2];
    // LDS stage of key tile t of the current item: by position in the workgroup's
    // sequence of key tiles over all its items (sq0: position of the item's first tile)
    int sq0 = 0;
    auto slot = [&](int t) __attribute__((always_inline)) { return PERS ? (sq0 + t - cur.tb) % NBUF : t % NBUF; };
    // loads of the tile 3 positions after t: past the item's last tile, CP takes the
    // next item's first tiles (when every item has at least 3 key tiles: P.cp)
    // (the SAFE redo never runs on: the next item then starts cold)
    auto load_next = [&](int t, auto safe_tag) __attribute__((always_inline)) {
        const int u = t + 3;
        if constexpr (decltype(safe_tag)::value) {
            load_raw(rk, rvr, u, safe_tag);
            return;
        }
        if constexpr (CP) {
            if (P.cp && has_nxt && u >= cur.te) {
                load_raw(nk, nv, nxt.tb + (u - cur.te), safe_tag);
                return;
            }
        }
        load_raw(rk, rv, u, safe_tag);
    };
    // Wave priority as in the 128-key steps (below): first half of the tile at 1, second
    // half at 0. For 8-wave D = 64 instances only: the D = 128 blocks (QK^T of the tile
    // at their start) ran 5-13% slower with it, the 2-wave ones 1.5%.
    constexpr bool PRIO_SPLIT = NW == 8 && D == 64;
    auto block = [&](int t, auto mask_tag, auto par_tag, auto safe_tag) __attribute__((always_inline)) {
        if constexpr (PRIO_SPLIT) __builtin_amdgcn_s_setprio(1);
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr int PC = PIPE2 ? decltype(par_tag)::value : 0;
        constexpr int PN = PIPE2 ? PC ^ 1 : 0;
        if constexpr (EARLY) {
            stage(slot(t + 2), safe_tag);
            load_next(t, safe_tag);
        }
        if constexpr (PIPE2)
            qk(slot(t + 1), sb[PN]);   // past the item's last tile: computed and unused
        else
            qk(slot(t), sb[0]);
        if constexpr (!MASK && FAST) {
            // Unmasked tile of a differential call: P against the current base, half by
            // half. A score more than ~16 above the base makes its P overflow fp16 to inf
            // (a row without a base yet has -m = +inf), which the row sum shows; only then
            // is the half redone with its exact maximum, O and l rescaled as in the masked
            // path. Most tiles so skip the maximum and the rescale of O.
            const uint16_t *Vt = smem + slot(t) * BUF_ELEMS + NBS * KS_ELEMS;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (PRIO_SPLIT && kb == 1) __builtin_amdgcn_s_setprio(0);
                u32x4 p[2];
                float part;
                softmax_half<false>(sb[PC][kb], kb, c, -st.m, TileMask{0, 0}, p, part);
                if (__builtin_expect(__any(!(part <= 3.0e38f)), 0)) {
                    const float mt = half_max(sb[PC][kb], c);
                    const float mn = (mt > st.m + TAU) ? mt : st.m;
                    const float ea = __builtin_amdgcn_exp2f(st.m - mn);
                    const float a = (mn == st.m) ? 1.0f : ea;
                    st.m = mn;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) st.o[db][i] *= a;
                    st.l *= a;
                    softmax_half<false>(sb[PC][kb], kb, c, (mn == NEG_INF) ? 0.0f : -mn, TileMask{0, 0}, p, part);
                }
                st.l += part;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        st.o[db] = mfma_pv(lds16(Vt + (db * 32 + r) * VT_STRIDE + kb * 32 + 16 * tt + 8 * g), p[tt],
                                           st.o[db]);
            }
            if constexpr (!EARLY) {
                stage(slot(t + 2), safe_tag);
                load_next(t, safe_tag);
            }
            __syncthreads();
            return;
        }
        if (MASK && tile_outside(t)) {
            if constexpr (!EARLY) {
                stage(slot(t + 2), safe_tag);
                load_next(t, safe_tag);
            }
            __syncthreads();
            return;
        }
        const TileMask mk = MASK ? tile_mask(t, L) : TileMask{0, 0};
        const float mt = tile_max<MASK>(sb[PC], c, mk);
        const float mn = (mt > st.m + TAU) ? mt : st.m;
        // branch-free: exp2(-inf) = 0 covers a row that had no valid key yet (the select
        // keeps the tile one basic block, which the scheduler can interleave)
        const float ea = __builtin_amdgcn_exp2f(st.m - mn);
        const float a = (mn == st.m) ? 1.0f : ea;
        st.m = mn;
        const float nb = (mn == NEG_INF) ? 0.0f : -mn;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) st.o[db][i] *= a;
        const uint16_t *Vt = smem + slot(t) * BUF_ELEMS + NBS * KS_ELEMS;
        float part[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (PRIO_SPLIT && kb == 1) __builtin_amdgcn_s_setprio(0);
            u32x4 p[2];
            softmax_half<false>(sb[PC][kb], kb, c, nb, mk, p, part[kb]);   // masked by tile_max
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    st.o[db] = mfma_pv(lds16(Vt + (db * 32 + r) * VT_STRIDE + kb * 32 + 16 * tt + 8 * g), p[tt],
                                       st.o[db]);
        }
        st.l = __builtin_fmaf(st.l, a, part[0] + part[1]);
        if constexpr (!EARLY) {
            stage(slot(t + 2), safe_tag);
            load_next(t, safe_tag);
        }
        __syncthreads();
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    auto step = [&](int t, auto par_tag, auto safe_tag) __attribute__((always_inline)) {
        if (tile_needs_mask(t, L))
            block(t, std::true_type{}, par_tag, safe_tag);
        else
            block(t, std::false_type{}, par_tag, safe_tag);
    };
    // ---- 128-key steps (PAIR) -------------------------------------------------------
    // The keys go in pairs of 64-key tiles (t, t+1), with one barrier per pair instead of
    // one per tile. The scores of a pair (four 32-key quarters) are computed during the
    // previous pair: each quarter's QK^T of the next pair is issued into the registers the
    // quarter's softmax has just freed, so its MFMAs run under the remaining softmax work.
    // Plain calls take one maximum over the pair's 128 scores, one move of the base and
    // one rescale of O per pair. Differential calls (FAST) compute each quarter's P
    // against the current base and redo a quarter with its exact maximum only when some P
    // overflowed, as the 64-key blocks do. K tile u sits in K-ring slot (u - tb) mod 4 and
    // V^T tile u in V-ring slot (u - tb) mod 4: the pair block of t reads K of t+2, t+3
    // and V of t, t+1, stages K of t+4, t+5 and V of t+2, t+3 (slots last read by the pair
    // block of t-2, closed by its barrier) from registers loaded during that block, and
    // loads K of t+6, t+7 and V of t+4, t+5. An item of an odd number of tiles ends with
    // one tile past its range, masked as keys past the item's end (kend).
    f32x16 sp[4];                             // scores of the current pair [tile][kb]
    u32x4 pk[2][NBS][KC], pv[2][VC];          // K' (each branch) / V' chunks of two tiles
    auto kring = [&](int t) __attribute__((always_inline)) {
        return smem + ((t - cur.tb) & (PR - 1)) * (NBS * KS_ELEMS);
    };
    auto vring = [&](int t) __attribute__((always_inline)) {
        return smem + PR * NBS * KS_ELEMS + ((t - cur.tb) & (PR - 1)) * VT_ELEMS;
    };
    auto pload_k = [&](int t, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KC; ++i)
#pragma unroll
            for (int br = 0; br < NBS; ++br) pk[j][br][i] = bload(rk[br], kl + (uint32_t)(t * BN + i * (NT / CPR)) * RB);
    };
    auto pload_v = [&](int t, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < VC; ++i) pv[j][i] = bload(rv, (uint32_t)t * (D * BN * 2) + (uint32_t)(tid + i * NT) * 16);
    };
    auto pstage_k = [&](int t, int j) __attribute__((always_inline)) {
        uint16_t *Ks = kring(t);
#pragma unroll
        for (int i = 0; i < KC; ++i)
#pragma unroll
            for (int br = 0; br < NBS; ++br)
                *reinterpret_cast<u32x4 *>(Ks + br * KS_ELEMS + kat + i * (NT / CPR) * KSTR) = pk[j][br][i];
    };
    auto pstage_v = [&](int t, int j) __attribute__((always_inline)) {
        uint16_t *Vt = vring(t);
#pragma unroll
        for (int i = 0; i < VC; ++i) {
            const int cv = tid + i * NT;
            *reinterpret_cast<u32x4 *>(Vt + (cv >> 3) * VT_STRIDE + (cv & 7) * 8) = pv[j][i];
        }
    };
    // S^T of one 32-key quarter (kb) of K tile t of this wave's branch
    auto qk_quarter = [&](int t, int kb, f32x16 &s) __attribute__((always_inline)) {
        const uint16_t *Ks = kring(t) + wbr * KS_ELEMS;
        u32x4 ka[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) ka[ks] = lds16(Ks + (kb * 32 + r) * KSTR + 16 * ks + 8 * g);
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc = mfma_qk<IO>(ka[ks], qreg[ks], acc);
        s = acc;
    };
    auto pv_quarter = [&](int t, int kb, const u32x4 (&p)[2]) __attribute__((always_inline)) {
        const uint16_t *Vt = vring(t);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                st.o[db] = mfma_pv(lds16(Vt + (db * 32 + r) * VT_STRIDE + kb * 32 + 16 * tt + 8 * g), p[tt], st.o[db]);
    };
    // Wave priority: the two waves of a SIMD run the same pair block, and the SIMD issues
    // for the older one first, which then idles at the barrier while the younger finishes
    // alone (27% of a pair, measured with per-wave clocks). A wave drops to the lower
    // priority for the second half of its pair (quarters 2 and 3), so the wave behind
    // gets the issue slots until it reaches that point too.
    auto pair_block = [&](int t, int kend, bool mask) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        pstage_k(t + 4, 0);
        pstage_k(t + 5, 1);
        pstage_v(t + 2, 0);
        pstage_v(t + 3, 1);
        pload_k(t + 6, 0);
        pload_k(t + 7, 1);
        pload_v(t + 4, 0);
        pload_v(t + 5, 1);
        // scores of keys past the item's end or outside the window set to -inf, in place
        // (a branch around this part only: the rest of the block is one copy of code)
        if (mask) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const TileMask mk = tile_mask(t + j, kend);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int o = kb * 32 + (i >> 2) * 8 + (i & 3);
                        sp[2 * j + kb][i] = ((uint32_t)(o - mk.lo) <= mk.span) ? sp[2 * j + kb][i] : NEG_INF;
                    }
            }
        }
        if constexpr (FAST) {
            // P of each quarter against the current base; a score more than ~16 above it
            // overflows fp16 to inf (a row without a base yet has -m = +inf), which the row
            // sum shows: only then is the quarter redone with its exact maximum
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int kb = q & 1;
                if (q == 2) __builtin_amdgcn_s_setprio(0);
                u32x4 p[2];
                float part;
                softmax_half<false>(sp[q], kb, c, -st.m, TileMask{0, 0}, p, part);
                if (__builtin_expect(__any(!(part <= 3.0e38f)), 0)) {
                    const float mt = half_max(sp[q], c);
                    const float mn = (mt > st.m + TAU) ? mt : st.m;
                    const float ea = __builtin_amdgcn_exp2f(st.m - mn);
                    const float a = (mn == st.m) ? 1.0f : ea;
                    st.m = mn;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) st.o[db][i] *= a;
                    st.l *= a;
                    softmax_half<false>(sp[q], kb, c, (mn == NEG_INF) ? 0.0f : -mn, TileMask{0, 0}, p, part);
                }
                st.l += part;
                qk_quarter(t + 2 + (q >> 1), kb, sp[q]);   // next pair: computed, unused past the item
                pv_quarter(t + (q >> 1), kb, p);
            }
        } else {
            // maximum of c * s over the pair's valid keys
            float v[2][32];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) v[j][kb * 16 + i] = sp[2 * j + kb][i];
            const float mr = pair_max(fmaxf(max32(v[0]), max32(v[1])));
            const float mt = (mr == NEG_INF) ? NEG_INF : mr * c;
            const float mn = (mt > st.m + TAU) ? mt : st.m;
            const float ea = __builtin_amdgcn_exp2f(st.m - mn);
            const float a = (mn == st.m) ? 1.0f : ea;
            const bool moved = mn != st.m;
            st.m = mn;
            const float nb = (mn == NEG_INF) ? 0.0f : -mn;
            // D = 128: the 64 multiplies only when some row's base moved (the factor is
            // otherwise exactly 1); at D = 64 the branch measured no faster
            if (D == 64 || __builtin_expect(__any(moved), 0)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) st.o[db][i] *= a;
            }
            float part[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int kb = q & 1;
                if (q == 2) __builtin_amdgcn_s_setprio(0);
                u32x4 p[2];
                softmax_half<false>(sp[q], kb, c, nb, TileMask{0, 0}, p, part[q]);   // masked above
                qk_quarter(t + 2 + (q >> 1), kb, sp[q]);   // next pair: computed, unused past the item
                pv_quarter(t + (q >> 1), kb, p);
            }
            st.l = __builtin_fmaf(st.l, a, (part[0] + part[1]) + (part[2] + part[3]));
        }
        __syncthreads();
    };

    // One pass over the current item: Q rotated into registers (MFMA B-operand layout),
    // O, l, m reset, the prologue when the item starts cold, then the key tiles.
    auto run_item = [&](auto safe_tag, bool cold, bool wait) __attribute__((always_inline)) {
        constexpr bool SAFE = decltype(safe_tag)::value;
        const int bb = cur.bh / P.H, hh = cur.bh - bb * P.H;
        const long long slab = (long long)cur.bh * L * D;   // contiguous offset of this (b, h)
        const rsrc_t rq = slab_rsrc(P.q, wbr * qbr + (CONTIG ? slab : bb * P.qb + hh * P.qh), qrb, L, RB);
        {
            const uint32_t row = (uint32_t)(qw + r);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const uint32_t col = (uint32_t)(16 * ks + 8 * g) * 2;
                if constexpr (CONTIG) {
                    const uint32_t offc = row * RB + col;
                    qreg[ks] = rope8<IO>(bload(rq, row * qrb + col), bload(rc, offc), bload(rs, offc)) ^ qsign;
                } else {
                    const RopeChunk rc8 = rope_chunk(2 * ks + g, rhalf, rdim);
                    const uint32_t to = rc8.mode ? row * trb + rc8.toff : NOWHERE;
                    const uint32_t t1 = rc8.mode >= 2 ? to + 16 : NOWHERE;
                    const uint32_t po = rc8.mode >= 2 ? row * qrb + (uint32_t)rc8.partner * 16 : NOWHERE;
                    qreg[ks] = rope8_general<IO>(bload(rq, row * qrb + col), bload(rq, po), bload(rc, to), bload(rc, t1),
                                                 bload(rs, to), bload(rs, t1), rc8.mode) ^ qsign;
                }
            }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) st.o[db] = f32x16{};
        st.l = 0.0f;
        st.m = NEG_INF;
        st.a = 1.0f;

        if constexpr (PAIR && !SAFE) {
            // (one item per workgroup: always cold) K of tb .. tb+3 and V of tb, tb+1 staged,
            // K of tb+4, tb+5 and V of tb+2, tb+3 loaded
            if (wait) __syncthreads();
            const int tb = cur.tb;
            pload_k(tb, 0);
            pload_k(tb + 1, 1);
            pload_v(tb, 0);
            pload_v(tb + 1, 1);
            pstage_k(tb, 0);
            pstage_k(tb + 1, 1);
            pstage_v(tb, 0);
            pstage_v(tb + 1, 1);
            pload_k(tb + 2, 0);
            pload_k(tb + 3, 1);
            pstage_k(tb + 2, 0);
            pstage_k(tb + 3, 1);
            pload_k(tb + 4, 0);
            pload_k(tb + 5, 1);
            pload_v(tb + 2, 0);
            pload_v(tb + 3, 1);
            __syncthreads();
            qk_quarter(tb, 0, sp[0]);
            qk_quarter(tb, 1, sp[1]);
            qk_quarter(tb + 1, 0, sp[2]);
            qk_quarter(tb + 1, 1, sp[3]);
            __syncthreads();   // every wave has read K of tb, tb+1 before the first pair block restages them
            const int kend = min(L, cur.te * BN);
            for (int t = cur.tb; t < cur.te; t += 2)
                pair_block(t, kend, tile_needs_mask(t, kend) || tile_needs_mask(t + 1, kend));
            return;
        }
        // ---- prologue: the first item, and every item without CP ------------------
        if (cold) {
            if (wait) __syncthreads();   // every wave is done with the LDS stages
            const rsrc_t &vv = SAFE ? rvr : rv;
            load_raw(rk, vv, cur.tb, safe_tag);
            stage(slot(cur.tb), safe_tag);
            load_raw(rk, vv, cur.tb + 1, safe_tag);
            stage(slot(cur.tb + 1), safe_tag);
            load_raw(rk, vv, cur.tb + 2, safe_tag);
            __syncthreads();
        }
        if constexpr (PIPE2) qk(slot(cur.tb), sb[0]);
        int t = cur.tb;
        for (; t + 1 < cur.te; t += 2) {
            step(t, P0{}, safe_tag);
            step(t + 1, P1{}, safe_tag);
        }
        if (t < cur.te) step(t, P0{}, safe_tag);
    };

    bool first = true, cold_next = false;
    for (;;) {
        const int bb = cur.bh / P.H, hh = cur.bh - bb * P.H;
        const long long slab = (long long)cur.bh * L * D;   // contiguous offset of this (b, h)
        const int q0 = cur.qt * BM;
        qw = q0 + wq * 32;
        qhi_live = min(qw + 31, L - 1);
        rvr = raw_v_of(cur.bh);
        run_item(std::false_type{}, first || cold_next || !(CP && P.cp), !first);
        first = false;
        cold_next = false;

        // ---- range guard of the bf16 -> fp16 V conversion (see attn_common.hpp) ------
        int vshift = 0;
        if constexpr (IO == IO_BF16) {
            if (__builtin_expect(wg_any<NW>(!acc_finite(st.o, st.l), guard), 0)) {
                // largest finite |v| over the key tiles this item visited
                uint32_t mx = 0;
                const int k_lo = cur.tb * BN, k_hi = min(cur.te * BN, L);
                for (int c = k_lo * CPR + tid; c < k_hi * CPR; c += NT)
                    mx = max(mx, bf16_finite_absmax(bload(rvr, (uint32_t)(c / CPR) * vrb + (uint32_t)(c % CPR) * 16)));
                vshift = vshift_of(wg_max<NW>(mx, guard + NW));
                if (vshift > 0) {
                    // redo the item with V scaled by 2^-vshift; the LDS stages and the
                    // registers CP filled for the next item are overwritten, so that one
                    // starts cold
                    vsc = exp2i(-vshift);
                    run_item(std::true_type{}, true, true);
                    cold_next = true;
                }
            }
        }

        // ---- split tail: hand this key range's (O, m, l) over, or merge them all --------
        // Every range stores its partial state (per wave and lane: O, m, l and the guard's
        // shift) and counts itself in; the workgroup that counts in last reads all the
        // partials and finishes the tile. Nobody waits. The partials are stored and read
        // as device-scope atomics, which the hardware keeps coherent across the XCDs'
        // L2 caches (a store completes at the device's coherence point: the wait for the
        // stores before the barrier orders them before the count); a device-scope fence
        // instead would write back and invalidate the whole L2, measured at 20-70 us.
        if constexpr (TAIL) {
            if (spl >= 0) {
                constexpr int ROWF = NDB * 16 + 4;   // floats per lane: O, m, l, shift, pad
                const int ns = P.n_split;
                auto slot_of = [&](int q) __attribute__((always_inline)) {
                    return P.part + ((long long)(spl * ns + q) * NW + wave) * (ROWF * 64) + lane;
                };
                auto put = [](float *p, float x) __attribute__((always_inline)) {
                    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                };
                auto get = [](const float *p) __attribute__((always_inline)) {
                    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                };
                float *mine = slot_of(part);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) put(mine + (db * 16 + i) * 64, st.o[db][i]);
                put(mine + (NDB * 16) * 64, st.m);
                put(mine + (NDB * 16 + 1) * 64, st.l);
                put(mine + (NDB * 16 + 2) * 64, __int_as_float(vshift));
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores are complete
                __syncthreads();
                if (tid == 0) guard[0] = __hip_atomic_fetch_add(P.cnt + spl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __syncthreads();
                if (guard[0] != (uint32_t)(ns - 1)) return;   // another range finishes the tile
                if (tid == 0) __hip_atomic_store(P.cnt + spl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // next call
                // the common base M and the common guard shift of all ranges, then their sum in
                // range order from the stored copies (the same operations whichever range
                // merges, so the result does not depend on which one finished last)
                float mx = NEG_INF;
                int vs = 0;
                for (int q = 0; q < ns; ++q) {
                    const float *th = slot_of(q);
                    mx = fmaxf(mx, get(th + (NDB * 16) * 64));
                    vs = max(vs, __float_as_int(get(th + (NDB * 16 + 2) * 64)));
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db) st.o[db] = f32x16{};
                st.l = 0.0f;
                for (int q = 0; q < ns; ++q) {
                    const float *th = slot_of(q);
                    const float mq = get(th + (NDB * 16) * 64);
                    // a range with no valid key for this row has m = -inf and weight 0
                    const float wq = mq == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(mq - mx);
                    const float vq = wq * exp2i(__float_as_int(get(th + (NDB * 16 + 2) * 64)) - vs);
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            st.o[db][i] = __builtin_fmaf(get(th + (db * 16 + i) * 64), vq, st.o[db][i]);
                    st.l = __builtin_fmaf(get(th + (NDB * 16 + 1) * 64), wq, st.l);
                }
                st.m = mx;
                vshift = vs;
            }
        }

        // ---- epilogue: normalise, subtract, cast, store rows < L -------------------------
        // (2^vshift undoes the guard's scaling of V; l >= 1, so inv * 2^vshift stays finite)
        const float inv = (1.0f / pair_sum(st.l)) * exp2i(vshift);
        const int qi = qw + r;
        if constexpr (DIFF) {
            // The second branch hands x2 = O2 / l2 to the first through LDS (the stages
            // are free once every wave has left the loop): element e of lane l of query
            // block wq at word (wq * 32 + e) * 64 + l, so a wave's 64 lanes write 64
            // consecutive words per element.
            float *xb = reinterpret_cast<float *>(smem + (CP ? NBUF * BUF_ELEMS : 0));
            __syncthreads();
            if (wbr == 1) {
    #pragma unroll
                for (int db = 0; db < NDB; ++db)
    #pragma unroll
                    for (int i = 0; i < 16; ++i) xb[(wq * 16 * NDB + db * 16 + i) * 64 + lane] = st.o[db][i] * inv;
            }
            __syncthreads();
        }
        if (!(DIFF && wbr == 1) && qi < L) {
        const long long row = CONTIG ? slab + (long long)qi * D : bb * P.ob + hh * P.oh + (long long)qi * P.ol;
        const float *xb = reinterpret_cast<const float *>(smem + (CP ? NBUF * BUF_ELEMS : 0));
    #pragma unroll
        for (int db = 0; db < NDB; ++db)
    #pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                float o[4];
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o[j] = st.o[db][grp * 4 + j] * inv;
                    if constexpr (DIFF) o[j] = o[j] - P.lam * xb[(wq * 16 * NDB + db * 16 + grp * 4 + j) * 64 + lane];
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

        // ---- next item ----------------------------------------------------------------
        if constexpr (!PERS) break;
        sq0 += cur.te - cur.tb;
        if (!has_nxt) break;
        item += (int)gridDim.x;
        cur = nxt;
#pragma unroll
        for (int br = 0; br < NBS; ++br) rk[br] = nk[br];
        rv = nv;
        has_nxt = item + (int)gridDim.x < n_items;
        if (has_nxt) {
            nxt = item_at(item + (int)gridDim.x);
            kv_of(nxt.bh, nk, nv);
        }
    }
}

// Query rows per workgroup of the 8-wave long-span instances.
int full_tile_rows(const LaunchArgs &a) {
    const int nw = a.D == 128 ? waves_for<128>() : waves_for<64>();
    return a.diff ? nw * 16 : nw * 32;
}

// Key tiles the widest query tile of `bm` rows spans.
long long key_span(const LaunchArgs &a, long long bm) {
    const long long all = ((long long)a.L + BN - 1) / BN;
    return a.window < 0 ? all : std::min(all, (2ll * a.window + bm + BN - 1) / BN + 1);
}

// Grids of more query tiles than compute units whose tiles span at most 32 key tiles:
// contiguous calls run them persistent (see launch_contig). A shape property, so that
// the workspace size (the split tail below) does not depend on the strides.
bool persistent_shape(const LaunchArgs &a) {
    if (use_narrow(a) || (a.prep && small_grid(a))) return false;
    const long long bm = full_tile_rows(a);
    const long long items = ((long long)a.L + bm - 1) / bm * a.B * a.H;
    return items > (a.n_cu > 0 ? a.n_cu : 256) && key_span(a, bm) <= 32;
}
bool runs_persistent(const LaunchArgs &a) { return a.contig && persistent_shape(a); }

template <int IO, bool DIFF, bool CONTIG, int D, bool PRE, bool PERS, int NW = waves_for<D>()>
hipError_t launch(const LaunchArgs &a, int n_qtiles) {
    Params P = make_params(a);
    P.n_qtiles = n_qtiles;
    P.n_items = n_qtiles * a.B * a.H;
    // persistent: at most one workgroup per compute unit (a multiple of 8, so that all
    // items of a workgroup fall on its XCD)
    const int ncu = a.n_cu >= 8 ? a.n_cu / 8 * 8 : 8;
    const unsigned grid = (unsigned)(PERS ? std::min(P.n_items, ncu) : P.n_items);
    // an item's key span is >= min(L, rows + w) keys, and >= 129 keys cover >= 3 tiles
    P.cp = (a.L >= 129 && (a.window < 0 || a.window >= 128)) ? 1 : 0;
    // the split tail runs its own instances, so that the others keep their code unchanged
    if constexpr (!PERS && PRE && NW == waves_for<D>()) {
        set_tail(P, a);
        if (P.n_split > 0) {
            hipLaunchKernelGGL((attn_fwd_kernel<IO, DIFF, CONTIG, D, PRE, PERS, NW, true>),
                               dim3((unsigned)(P.n_full + P.n_tail * P.n_split)), dim3(NW * 64), 0,
                               static_cast<hipStream_t>(a.stream), P);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((attn_fwd_kernel<IO, DIFF, CONTIG, D, PRE, PERS, NW>), dim3(grid), dim3(NW * 64), 0,
                       static_cast<hipStream_t>(a.stream), P);
    return hipGetLastError();
}

// Grids of more query tiles than compute units run persistent (contiguous instances):
// the pipeline of key tiles then runs on from one query tile of a workgroup into the
// next, which hides the next tile's start behind the current tile's last blocks.
// Measured: 8% faster at a differential window of half-width 256 (10 key tiles per
// query tile), within 1% at 64 key tiles (the start is a small share there, and the
// bookkeeping costs ~30 scalar instructions per tile), so up to 32 key tiles.
template <int IO, bool DIFF, int D, bool PRE>
hipError_t launch_contig(const LaunchArgs &a, int n_qtiles) {
    if constexpr (PRE && !DIFF && D == 64)
        if (small_grid(a)) return launch<IO, false, true, 64, true, false, 2>(a, n_qtiles);
    if (runs_persistent(a)) return launch<IO, DIFF, true, D, PRE, true>(a, n_qtiles);
    return launch<IO, DIFF, true, D, PRE, false>(a, n_qtiles);
}

template <int IO, int D, bool PRE>
hipError_t launch_io(const LaunchArgs &a, int n_qtiles) {
    if (a.contig) return a.diff ? launch_contig<IO, true, D, PRE>(a, n_qtiles) : launch_contig<IO, false, D, PRE>(a, n_qtiles);
    if constexpr (PRE && D == 64)
        if (small_grid(a)) return launch<IO, false, false, 64, true, false, 2>(a, n_qtiles);
    return a.diff ? launch<IO, true, false, D, PRE, false>(a, n_qtiles) : launch<IO, false, false, D, PRE, false>(a, n_qtiles);
}

template <int D>
hipError_t launch_d(const LaunchArgs &a, int n_qtiles) {
    if (a.dtype == 1) return a.prep ? launch_io<IO_BF16, D, true>(a, n_qtiles) : launch_io<IO_BF16, D, false>(a, n_qtiles);
    return a.prep ? launch_io<IO_F16, D, true>(a, n_qtiles) : launch_io<IO_F16, D, false>(a, n_qtiles);
}

}  // namespace

// Sequences of at most 256 keys and windows of half-width <= 32 go to the single-span
// kernel (attn_narrow.hip), which stages a query block's whole key span at once; it is
// built for D = 64 only, so D = 128 always takes the long-span kernel.
bool use_narrow(const LaunchArgs &a) { return a.D == 64 && narrow_applies(a); }

// Plain calls at D = 64 whose grid of 256-row query tiles leaves compute units
// idle (fewer workgroups than compute units, e.g. B=1 H=24 L=1292: 144 workgroups on
// 256 CUs) run 64-row tiles on the pre-pass workspace (AUTO runs the pre-pass for
// them, prep_pays): full attention on contiguous tensors in the key-split kernel
// (attn_split.hip: 4 waves, each key half of a tile on its own pair of waves, so every
// SIMD runs two waves), other such calls as 2-wave workgroups of this kernel, two per
// compute unit (one wave per SIMD, every CU busy). Without the pre-pass either would
// rotate and transpose each key tile for only 64 rows.
// Only grids whose 64-row tiles fit in one round of two workgroups per compute unit:
// measured on B=1 H=24, L = 2000 (768 workgroups of 64 rows, 1.5 rounds) the 256-row
// tiles of the fused path are 10% faster.
bool small_grid(const LaunchArgs &a) {
    if (a.D != 64 || a.diff || use_narrow(a)) return false;
    const long long bh = (long long)a.B * a.H;
    return ((long long)a.L + 255) / 256 * bh < a.n_cu && ((long long)a.L + 63) / 64 * bh <= 2ll * a.n_cu;
}

// Query rows per workgroup: 32 per wave plain, 32 per pair of waves differential.
int tile_rows(const LaunchArgs &a) {
    if (use_narrow(a)) return narrow_tile_rows(a);
    if (a.prep && small_grid(a)) return 64;
    const int nw = a.D == 128 ? waves_for<128>() : waves_for<64>();
    return a.diff ? nw * 16 : nw * 32;
}

// The split tail. A one-round-per-tile grid (8-wave workgroups, one per compute unit)
// whose last round holds r <= CUs / 2 query tiles would run that round with most CUs
// idle: instead each of those r tiles is split into k = min(4, CUs / r) contiguous key
// ranges (at least 4 key tiles each), one workgroup per range, and the workgroup that
// finishes a tile's last range merges the ranges' partial (O, m, l) from the workspace
// (O = sum of 2^(m_i - M) O_i, l likewise, M the largest base), so the last round takes
// about 1/k of a tile's time. Grids of fewer tiles than half the CUs split all of them.
// Not for the shapes of the persistent and small-grid instances, which have their own
// balance (strided calls of a persistent shape run one round per tile without a split).
TailPlan tail_plan(const LaunchArgs &a) {
    const unsigned long long lp = ((unsigned long long)a.L + BN - 1) / BN * BN;
    const unsigned long long kv = (unsigned long long)(a.diff ? 3 : 2) * (unsigned long long)a.B *
                                  (unsigned long long)a.H * lp * (unsigned long long)a.D * 2ull;
    TailPlan t{0, 0, 0, kv, kv, kv};
    if (!a.tail_ok || use_narrow(a) || small_grid(a) || persistent_shape(a)) return t;
    const long long bm = full_tile_rows(a);
    const long long items = ((long long)a.L + bm - 1) / bm * a.B * a.H;
    const long long ncu = a.n_cu > 0 ? a.n_cu : 256;
    const long long rem = items % ncu;
    if (rem == 0 || 2 * rem > ncu) return t;
    const long long span = key_span(a, bm);
    long long k = std::min(4ll, ncu / rem);
    while (k > 1 && span < 4 * k) --k;
    if (k < 2) return t;
    t.n_full = (int)(items - rem);
    t.k = (int)k;
    t.n_tail = (int)rem;
    // per range: 8 waves x 64 lanes x (O, m, l, shift, pad) floats
    const unsigned long long rowf = (unsigned long long)a.D / 32 * 16 + 4;
    t.cnt_off = kv + (unsigned long long)rem * k * 8ull * rowf * 64ull * 4ull;
    t.end = t.cnt_off + ((unsigned long long)rem * 4ull + 255ull) / 256ull * 256ull;
    return t;
}

// Workspace of the pre-pass: K' of each branch and V', Lp x D 16-bit values per (b, h)
// each, then the split tail's partials and counters when it applies (0 for calls that
// take the single-span kernel).
unsigned long long prep_bytes(const LaunchArgs &a) {
    if (use_narrow(a)) return 0;
    return tail_plan(a).end;
}

// The fused staging rotates and transposes a key tile once per query tile that visits
// it; the pre-pass does that once but adds a pass over K and V (about one more read and
// write of each) before the attention kernel can start. Measured (always against never,
// same process, 21 shapes, with the 128-key steps and the split tail in place):
//  * D = 128: the pre-pass wins on every shape, 18-35% (windows of half-width 256 to
//    1024 at 4-10 visits, persistent or not, plain and differential; full attention at
//    L = 2048 in one round): its fused staging rotates 128 dims per key and its
//    instances spill.
//  * D = 64, grids that run one round per tile (the pair steps): from about 10 visits
//    plain (a 1024-key window, 10 visits: 8% faster; L = 2048 in one round, 8 visits:
//    even) and 18 differential: once the fused 64-key blocks skipped the window tiles
//    outside a wave's rows, they won the one-round differential windows up to ~17 visits
//    (B=1 H=8 L=4096: 10 visits 12% faster than the pre-pass, 14 visits 3.5%, 18 even;
//    26 visits and full attention, 32, 6-10% slower), in one round or several.
//  * D = 64 persistent grids (windows whose tiles span <= 32 key tiles): from 12 visits
//    plain and 9 differential (plain 768-key window, 8 visits: 1% slower; differential
//    1024-key window, 10 visits: 1% faster, 1536: 5% faster; 256, 6 visits: 7% slower).
bool prep_pays(const LaunchArgs &a) {
    if (use_narrow(a)) return false;
    if (small_grid(a)) return true;
    // the split tail needs the workspace, and a last round of at most half the CUs split
    // into k ranges measured 10-49% faster than that round whole (even at 4 key tiles
    // per range: B=1 H=2 L=1000 differential, 0.0305 -> 0.0226 ms)
    if (tail_plan(a).k > 0) return true;
    const int bm = tile_rows(a);
    const long long n_qtiles = ((long long)a.L + bm - 1) / bm;
    const long long visits = a.window < 0 ? n_qtiles : std::min(n_qtiles, (2ll * a.window + BN + bm - 1) / bm + 1);
    if (a.D == 128) return visits >= 3;
    // A workspace query does not know the strides (contig is 0 there), so for a shape that
    // runs persistent when contiguous the answer must cover the contiguous call: the
    // differential threshold is the persistent one whatever the strides, and the plain
    // one for strided calls (10) is below the persistent one (12).
    if (persistent_shape(a)) return visits >= (a.diff ? 9 : a.contig ? 12 : 10);
    return visits >= (a.diff ? 18 : 10);
}

int launch_forward(const LaunchArgs &a) {
    if (use_narrow(a)) return a.run_main ? launch_narrow(a) : (int)hipSuccess;
    if (a.prep && a.run_prep) {
        const int e = launch_prep(a);
        if (e != (int)hipSuccess) return e;
    }
    if (!a.run_main) return (int)hipSuccess;
    const int bm = tile_rows(a);
    const int n_qtiles = (a.L + bm - 1) / bm;
    if (a.prep && small_grid(a) && split_applies(a)) return launch_split(a, n_qtiles);
    return (int)(a.D == 128 ? launch_d<128>(a, n_qtiles) : launch_d<64>(a, n_qtiles));
}

}  // namespace sa3
