// Fused RoPE attention forward on gfx950 for key spans short enough to stage at once:
// narrow sliding windows (half-width w <= 32; the SAME-L decoder's own window is +-17
// keys, TensorRT engines README, section "Building your own"; "How the kernels differ"
// for the differential form) and short sequences (L <= 256: the short latents of the
// DiTs, sa3_trt README, section "DiT precision").
//
// With so few keys per query the work is bound by HBM traffic and load latency, not
// by the MFMA: the long-span kernel's four-stage software pipeline would mostly run
// its prologue. Here one workgroup takes a short block of query rows and stages the
// whole key span they can see at once ([q0 - w, q0 + BM - 1 + w], BM + 64 keys, for a
// narrow window; all of [0, L) for a short sequence), then each wave computes its
// scores over its part of that span (for a window, the three 32-key blocks its rows can
// see), one exact softmax (the maximum over those keys is known, so there is no running
// rescale), and P.V, and stores. Small workgroups and a small
// LDS footprint keep several of them resident per CU so that their loads overlap.
//
//  * Plain, windowed: 4 waves x 32 query rows (BM = 128); span 192 keys. The
//    workgroup's Q rows (each branch) are loaded with whole rows per wave load and
//    rotated once into LDS, where each wave reads its B operands before the span is
//    staged over them.
//  * Plain, short sequence: the waves split the span instead of the rows, each taking
//    32 of its keys (KSPLIT = 2 waves per 32-row block at 64 keys, BM = 64; 4 waves at
//    128 keys and 8 waves at 256, BM = 32): each wave takes its share of the keys for
//    its block's 32 rows with its own exact maximum, row sum and O, and the shares are
//    merged through LDS at the end (O = sum of 2^(m_w - M) O_w, l likewise, M the
//    largest m_w), each wave merging and storing its part of the O elements. A 256-key
//    sequence then runs 8 query tiles per head instead of 2, which fills 4x more CUs.
//    The workgroup's query rows are loaded and rotated once (whole rows per wave load)
//    into LDS, from which each wave reads its B operands.
//  * Differential: waves w and w + 2 share 32 rows, one softmax branch each (BM = 64),
//    windowed span 128 keys; the second branch hands O2 / l2 to the first through LDS.
//  * Arithmetic per element is the long-span kernel's: RoPE in FP32 with separate
//    roundings then RNE to the IO dtype, S^T = K Q^T on MFMA (FP32 accumulation),
//    P = 2^(s * c - m) rounded to fp16, FP32 row sums of the rounded P, O^T = V^T P^T
//    on MFMA with V in fp16, out = O / l (minus lambda * O2 / l2 in FP32).
//  * Keys before 0 or at / after L read as zeros through the buffer range check (a
//    negative row gives an offset far above num_records) and are masked.

#include "attn_common.hpp"

namespace sa3 {
namespace {

// Span of keys staged per workgroup and the LDS strides (16-bit elements). NKF = 0:
// windowed mode, the span [q0 - w, q0 + BM - 1 + w] of a window of half-width w <= 32
// (BM + 64 keys). NKF > 0: short-sequence mode, the whole sequence [0, L) with L <= NKF
// and any window. The V^T stride keeps the 16-byte operand reads of 16 consecutive
// rows on distinct banks. The K rows are padded to 72 elements for the same purpose,
// except in the differential windowed mode, whose 53 KB would then miss three
// workgroups per CU (LDS is granted in 2 KB units): there the rows are 64 elements
// and the 16-byte chunk c of row k is stored at chunk c ^ (k & 7), which puts any 8
// consecutive rows' reads of one chunk, and one row's 8 chunk writes, on distinct
// banks without the padding.
template <bool DIFF, int NKF>
struct NarrowShape {
    // threads: 4 waves, or 8 for the plain 256-key span (one 32-key share each: twice the
    // threads for its staging, which with one wave per SIMD was issue-bound)
    static constexpr bool W8 = !DIFF && NKF == 256;
    static constexpr int NT = W8 ? 512 : 256;
    static constexpr int NBS = DIFF ? 2 : 1;          // branches staged
    // waves per 32-row query block (one 32-key share each)
    static constexpr int KSPLIT = (DIFF || NKF == 0) ? 1 : NKF == 64 ? 2 : NT / 64;
    static constexpr int WPB = DIFF ? 2 : (NT / 64) / KSPLIT; // query blocks per branch
    static constexpr int BM = WPB * 32;               // query rows per workgroup
    static constexpr int NK = NKF ? NKF : BM + 64;    // keys staged
    static constexpr int NKB = NK / 32;               // 32-key blocks
    static constexpr bool SWZ = DIFF && NKF == 0;     // swizzled, unpadded K rows
    static constexpr int KS = SWZ ? 64 : 72;          // K row stride
    static constexpr int VS = NK + 8;                 // V^T row stride
    static constexpr int K_ELEMS = NK * KS;
    static constexpr int V_ELEMS = HD * VS;
    static constexpr int LDS_ELEMS = NBS * K_ELEMS + V_ELEMS;
};

// Windowed mode keeps registers <= 168 so that three workgroups share a CU (their LDS
// fits too); short-sequence mode and the general instances may use up to 256; the
// 256-key span runs one workgroup per CU (up to 512 registers for the 4-wave
// differential one, 256 for the 8-wave plain one).
// CONTIG: contiguous [B][H][L][64] tensors (q, k stacked [2][...]); the row strides
// are then compile-time constants.
template <int IO, bool DIFF, int NKF, bool CONTIG>
__global__ __launch_bounds__((NarrowShape<DIFF, NKF>::NT), (NKF == 256) ? 1 : (CONTIG && !NKF) ? 3 : 2) void attn_narrow_kernel(Params P) {
    using S = NarrowShape<DIFF, NKF>;
    constexpr int NT = S::NT, NBS = S::NBS, WPB = S::WPB, BM = S::BM, NK = S::NK, NKB = S::NKB;
    constexpr int KSPLIT = S::KSPLIT;
    // 32-key blocks a wave computes: its share of the span in short-sequence mode; in
    // windowed mode the three blocks from its own row offset, which hold every key its 32
    // rows can see (offsets 32 wq .. 32 wq + 31 + 2w of the span, w <= 32); the span's
    // other blocks are wholly outside its rows' windows
    constexpr int NKBW = NKF ? NKB / KSPLIT : 3;
    static_assert(NKF || (WPB - 1) + NKBW <= NKB, "windowed blocks inside the span");
    static_assert(NKB % KSPLIT == 0, "key split");
    // the merge of the key shares reuses the staging area: NT / 64 waves x 34 rows of 64 floats
    constexpr int MERGE_ELEMS = KSPLIT > 1 ? (NT / 64) * 34 * 64 * 2 : 0;
    // QCOOP: short sequences split over the waves (several waves on the same 32 query
    // rows) load and rotate the workgroup's rows once, 16-byte chunks m = tid + NT i (row
    // m / 8) with whole rows per wave load, into LDS after the span (QS-element rows), and
    // each wave reads its B operands from there
    constexpr bool QCOOP = KSPLIT > 1 && CONTIG;
    constexpr bool QWIN = NKF == 0 && CONTIG;
    constexpr int QS = 72;
    constexpr int Q_ELEMS = QCOOP ? BM * QS : 0;
    constexpr int QCH = (BM * 8 + NT - 1) / NT;   // Q chunks per thread (QCOOP)
    static_assert(!QCOOP || BM * 8 <= NT * QCH, "Q chunks");
    static_assert(!QWIN || (BM * 8 % NT == 0 && NBS * BM * QS <= NBS * S::K_ELEMS), "Q rows in the K area");
    constexpr int SMEM_ELEMS = S::LDS_ELEMS + Q_ELEMS > MERGE_ELEMS ? S::LDS_ELEMS + Q_ELEMS : MERGE_ELEMS;
    constexpr int KC = NK * 8 / NT;          // K chunks (8 elements) per thread per branch
    constexpr int VC = NK * 4 / NT;          // V items (2 keys x 8 d) per thread
    static_assert(NK * 8 % NT == 0 && NK * 4 % NT == 0, "staging split");
    static_assert(!DIFF || S::LDS_ELEMS * 2 >= WPB * 32 * 64 * 4, "LDS too small for the O2 exchange");
    __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
    __shared__ uint32_t guard[2 * (NT / 64)];   // words of the V range guard's reductions

    const float NEG_INF = -__builtin_inff();
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wbr = DIFF ? wave / WPB : 0;
    const int wq = DIFF ? wave % WPB : wave / KSPLIT;
    const int kq = DIFF ? 0 : wave % KSPLIT;  // this wave's share of the span
    const int r = lane & 31;
    const int g = lane >> 5;
    const int L = P.L;
    const int w = P.window;
    const float c = P.c;

    // XCD-aware remap of the workgroup id, as in the long-span kernel.
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int per = nblk >> 3, rem = nblk & 7, xcd = bid & 7, idx = bid >> 3;
    const int lid = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    // windowed mode: query tiles major, heads minor, so the workgroups an XCD runs at
    // once share the rows of the cos/sin table (and a head's neighbouring tiles, their
    // halos); a short sequence keeps each head's workgroups together (the whole span)
    const int nbh = nblk / P.n_qtiles;
    const int bh = NKF ? lid / P.n_qtiles : lid % nbh;
    const int qt = NKF ? lid - bh * P.n_qtiles : lid / nbh;

    const int bb = bh / P.H, hh = bh - bb * P.H;
    const uint32_t qrb = CONTIG ? (uint32_t)ROWB : P.q_rowb;
    const uint32_t krb = CONTIG ? (uint32_t)ROWB : P.k_rowb;
    const uint32_t vrb = CONTIG ? (uint32_t)ROWB : P.v_rowb;
    const long long slab = (long long)bh * L * HD;   // contiguous offset of this (b, h)
    const long long qbr = CONTIG ? (long long)(nblk / P.n_qtiles) * L * HD : P.q_br;
    const long long kbr = CONTIG ? qbr : P.k_br;
    rsrc_t rk[NBS];
#pragma unroll
    for (int br = 0; br < NBS; ++br)
        rk[br] = slab_rsrc(P.k, br * kbr + (CONTIG ? slab : bb * P.kb + hh * P.kh), krb, L);
    const rsrc_t rq = slab_rsrc(P.q, wbr * qbr + (CONTIG ? slab : bb * P.qb + hh * P.qh), qrb, L);
    const rsrc_t rv = slab_rsrc(P.v, CONTIG ? slab : bb * P.vb + hh * P.vh, vrb, L);
    // cos/sin: [L][R/2] floats (R = 64 in the contiguous instances: 128 bytes per row)
    const uint32_t trb = CONTIG ? (uint32_t)ROWB : P.tab_rowb;
    const rsrc_t rc = make_rsrc(P.cos, (uint32_t)L * trb);
    const rsrc_t rs = make_rsrc(P.sin, (uint32_t)L * trb);
    const int rhalf = P.rope_half, rdim = P.rot_dim;
    constexpr uint32_t NOWHERE = 0xfffffff0u;   // an offset past every buffer: reads zeros

    const int q0 = qt * BM;
    const int qw = q0 + wq * 32;
    const int ks0 = NKF ? 0 : q0 - w;        // first staged key (may be negative)

    // One pass: issue every load (Q rows of this wave, then the K / cos / sin / V span),
    // stage, and compute this wave's O, l and maximum. SAFE: the redo of the V range
    // guard (bf16 only), which scales V by vsc = 2^-shift as it converts it.
    const int qi = qw + r;
    f32x16 o[2];
    float l, mx;
    float vsc = 1.0f;
    // V item it -> keys 2p, 2p + 1 of the span and 8 values of d from 8 ch. Consecutive
    // lanes take consecutive 16-byte chunks of one key row (ch fastest), so that a wave's
    // loads cover whole 128-byte rows instead of 16 bytes of each of 64 rows (samel_w17 6%,
    // the 128-key graph calls 3.5% faster); a 64-key span keeps p fastest (its one item per
    // thread measured 0.5-1.3% slower either way).
    auto v_item = [](int it, int &p, int &ch) __attribute__((always_inline)) {
        if constexpr (NKF == 64) {
            p = it % (NK / 2);
            ch = it / (NK / 2);
        } else {
            p = it / 8;
            ch = it % 8;
        }
    };
    // V^T element (row d, key position e) of the staged span. At a 256-key span the
    // 16-byte chunk e / 8 of row d sits at chunk (e / 8) ^ ((d / 8) & 7): the transposing
    // writes of one key row's chunks (lanes eight rows of V^T apart, whose rows' stride is
    // a multiple of 128 bytes) then fall in different banks, and the P.V operand reads
    // (rows of one 8-row group share the XOR) stay conflict-free; the 256-key graph calls
    // 5% faster. Elsewhere the plain layout measured the same or better.
    auto vt_off = [](int d, int e) __attribute__((always_inline)) {
        if constexpr (NKF == 256)
            return d * S::VS + ((((e >> 3) ^ (d >> 3)) & 7) | ((e >> 3) & ~7)) * 8 + (e & 7);
        else
            return d * S::VS + e;
    };
    auto compute = [&](auto safe_tag) __attribute__((always_inline)) {
        constexpr bool SAFE = decltype(safe_tag)::value;
        // The redo derives its lane values from an opaque copy of the thread id, so that the
        // compiler cannot share address arithmetic between the two passes (which would keep
        // it in registers through the first one).
        int tid = (int)threadIdx.x;
        if constexpr (SAFE) __asm__ volatile("" : "+v"(tid));
        const int lane = tid & 63, r = lane & 31, g = lane >> 5;
        const int qi = qw + r;
        // Q: the rotated chunks go straight to registers; general instances also load the
        // partner chunks and table floats 4-7 (half-split pairs)
        u32x4 qreg[4];
        const uint32_t qsign = P.neg_scale ? 0x80008000u : 0u;
        u32x4 rq_raw[4], rqc[4], rqs[4];
        // QWIN: windowed workgroups (each wave its own 32 rows of one branch) load their Q
        // rows once for the workgroup with whole rows per wave load (one (row, chunk) of both
        // branches per thread and item), rotate them into LDS at the start of the K area,
        // and each wave reads its B operands from there before the span is staged over it
        constexpr int QN = QWIN ? BM * 8 / NT : 1;
        u32x4 wq_raw[QN][NBS], wq_c[QN], wq_s[QN];
        if constexpr (QWIN) {
#pragma unroll
            for (int i = 0; i < QN; ++i) {
                const int m = tid + NT * i;
                const uint32_t row = (uint32_t)(q0 + m / 8), col = (uint32_t)(m % 8) * 16;
#pragma unroll
                for (int br = 0; br < NBS; ++br) {
                    const rsrc_t rqb = slab_rsrc(P.q, br * qbr + slab, qrb, L);
                    wq_raw[i][br] = bload(rqb, row * qrb + col);
                }
                wq_c[i] = bload(rc, row * ROWB + col);
                wq_s[i] = bload(rs, row * ROWB + col);
            }
        } else if constexpr (QCOOP) {
            // chunk m = tid + NT i of the workgroup's BM rows (row q0 + m / 8); with fewer
            // chunks than threads, the first BM * 8 threads hold them
#pragma unroll
            for (int i = 0; i < QCH; ++i) {
                const int m = tid + NT * i;
                if (BM * 8 >= NT * (i + 1) || m < BM * 8) {
                    const uint32_t row = (uint32_t)(q0 + m / 8), col = (uint32_t)(m % 8) * 16;
                    rq_raw[i] = bload(rq, row * qrb + col);
                    rqc[i] = bload(rc, row * ROWB + col);
                    rqs[i] = bload(rs, row * ROWB + col);
                }
            }
        } else {
            const uint32_t row = (uint32_t)(qw + r);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const uint32_t col = (uint32_t)(16 * ks + 8 * g) * 2;
                rq_raw[ks] = bload(rq, row * qrb + col);
                if constexpr (CONTIG) {
                    rqc[ks] = bload(rc, row * ROWB + col);
                    rqs[ks] = bload(rs, row * ROWB + col);
                } else {
                    const RopeChunk rc8 = rope_chunk(2 * ks + g, rhalf, rdim);
                    const uint32_t to = rc8.mode ? row * trb + rc8.toff : NOWHERE;
                    const uint32_t t1 = rc8.mode >= 2 ? to + 16 : NOWHERE;
                    const uint32_t po = rc8.mode >= 2 ? row * qrb + (uint32_t)rc8.partner * 16 : NOWHERE;
                    qreg[ks] = rope8_general<IO>(rq_raw[ks], bload(rq, po), bload(rc, to), bload(rc, t1), bload(rs, to),
                                                 bload(rs, t1), rc8.mode) ^ qsign;
                }
            }
        }
        // K item i: span row (tid >> 3) + i * NT / 8, chunk tid & 7. The per-lane part of
        // the offset is one multiply here; the per-item part is wave-uniform (scalar unit).
        u32x4 rawk[NBS][KC], rawc[KC], raws[KC];
        u32x4 rawp[CONTIG ? 1 : NBS][CONTIG ? 1 : KC], rawc1[CONTIG ? 1 : KC], raws1[CONTIG ? 1 : KC];
        const RopeChunk kch = rope_chunk(tid & 7, rhalf, rdim);
        const uint32_t kl = (uint32_t)(tid >> 3) * krb + (uint32_t)(tid & 7) * 16;
        const uint32_t kpl = (uint32_t)(tid >> 3) * krb + (uint32_t)kch.partner * 16;
        const uint32_t cl = CONTIG ? (uint32_t)(tid >> 3) * ROWB + (uint32_t)(tid & 7) * 16
                                   : (uint32_t)(tid >> 3) * trb + kch.toff;
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const uint32_t r0 = (uint32_t)(ks0 + i * (NT / 8));
#pragma unroll
            for (int br = 0; br < NBS; ++br) rawk[br][i] = bload(rk[br], kl + r0 * krb);
            if constexpr (CONTIG) {
                rawc[i] = bload(rc, cl + r0 * ROWB);
                raws[i] = bload(rs, cl + r0 * ROWB);
            } else {
                const uint32_t to = kch.mode ? cl + r0 * trb : NOWHERE;
                const uint32_t t1 = kch.mode >= 2 ? to + 16 : NOWHERE;
                const uint32_t po = kch.mode >= 2 ? kpl + r0 * krb : NOWHERE;
#pragma unroll
                for (int br = 0; br < NBS; ++br) rawp[br][i] = bload(rk[br], po);
                rawc[i] = bload(rc, to);
                raws[i] = bload(rs, to);
                rawc1[i] = bload(rc, t1);
                raws1[i] = bload(rs, t1);
            }
        }
        // V item: keys 2p, 2p + 1 of the span and 8 values of d from 8 * ch
        u32x4 rawv[VC][2];
#pragma unroll
        for (int i = 0; i < VC; ++i) {
            const int it = tid + NT * i;
            int p, ch;
            v_item(it, p, ch);
            const uint32_t off = (uint32_t)(ks0 + 2 * p) * vrb + (uint32_t)ch * 16;
            rawv[i][0] = bload(rv, off);
            rawv[i][1] = bload(rv, off + vrb);
        }

        // ---- rotate Q into registers; rotate / transpose the span into LDS ---------------
        if constexpr (QWIN) {
#pragma unroll
            for (int i = 0; i < QN; ++i) {
                const int m = tid + NT * i;
#pragma unroll
                for (int br = 0; br < NBS; ++br)
                    *reinterpret_cast<u32x4 *>(smem + (br * BM + m / 8) * QS + (m % 8) * 8) =
                        rope8<IO>(wq_raw[i][br], wq_c[i], wq_s[i]) ^ qsign;
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qreg[ks] = lds16(smem + (wbr * BM + wq * 32 + r) * QS + 16 * ks + 8 * g);
            __syncthreads();   // every wave has its Q before the span is staged over it
        } else if constexpr (QCOOP) {
#pragma unroll
            for (int i = 0; i < QCH; ++i) {
                const int m = tid + NT * i;
                if (BM * 8 >= NT * (i + 1) || m < BM * 8)
                    *reinterpret_cast<u32x4 *>(smem + S::LDS_ELEMS + (m / 8) * QS + (m % 8) * 8) =
                        rope8<IO>(rq_raw[i], rqc[i], rqs[i]) ^ qsign;
            }
        } else if constexpr (CONTIG) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qreg[ks] = rope8<IO>(rq_raw[ks], rqc[ks], rqs[ks]) ^ qsign;
        }
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int it = tid + NT * i;
            const int at = (it >> 3) * S::KS + ((it & 7) ^ (S::SWZ ? (it >> 3) & 7 : 0)) * 8;
#pragma unroll
            for (int br = 0; br < NBS; ++br) {
                u32x4 rot;
                if constexpr (CONTIG)
                    rot = rope8<IO>(rawk[br][i], rawc[i], raws[i]);
                else
                    rot = rope8_general<IO>(rawk[br][i], rawp[br][i], rawc[i], rawc1[i], raws[i], raws1[i], kch.mode);
                *reinterpret_cast<u32x4 *>(smem + br * S::K_ELEMS + at) = rot;
            }
        }
        uint16_t *Vt = smem + NBS * S::K_ELEMS;
#pragma unroll
        for (int i = 0; i < VC; ++i) {
            const int it = tid + NT * i;
            int p, ch;
            v_item(it, p, ch);
            // key positions inside each 16 carry bits 2 and 3 swapped (the P.V operand order)
            const int k2 = 2 * p;
            const int pos = (k2 & ~12) | ((k2 & 4) << 1) | ((k2 & 8) >> 1);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t wa = rawv[i][0][j >> 1], wb = rawv[i][1][j >> 1];
                uint32_t wv;
                if constexpr (IO == IO_BF16) {
                    float fa = __uint_as_float((j & 1) ? (wa & 0xffff0000u) : (wa << 16));
                    float fb = __uint_as_float((j & 1) ? (wb & 0xffff0000u) : (wb << 16));
                    if constexpr (SAFE) {
                        fa *= vsc;
                        fb *= vsc;
                    }
                    wv = pack2<IO_F16>(fa, fb);
                } else {
                    wv = (j & 1) ? __builtin_amdgcn_perm(wb, wa, 0x07060302u) : __builtin_amdgcn_perm(wb, wa, 0x05040100u);
                }
                *reinterpret_cast<uint32_t *>(Vt + vt_off(8 * ch + j, pos)) = wv;
            }
        }
        __syncthreads();
        if constexpr (QCOOP) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qreg[ks] = lds16(smem + S::LDS_ELEMS + ((WPB == 1 ? 0 : wq) * 32 + r) * QS + 16 * ks + 8 * g);
        }

        // ---- scores of this wave's 32 rows over the span: S^T blocks of 32 keys ----------
        const uint16_t *Ks = smem + wbr * S::K_ELEMS;
        // s[j]: keys of 32-key block kb = kb0 + j of the span
        const int kb0 = NKF ? kq * NKBW : wq;
        f32x16 s[NKBW];
#pragma unroll
        for (int j = 0; j < NKBW; ++j) {
            const int kb = kb0 + j;
            u32x4 ka[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                ka[ks] = lds16(Ks + (kb * 32 + r) * S::KS + ((2 * ks + g) ^ (S::SWZ ? r & 7 : 0)) * 8);
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) acc = mfma_qk<IO>(ka[ks], qreg[ks], acc);
            s[j] = acc;
        }

        // valid keys of this lane's query: [max(0, qi - w), min(L - 1, qi + w)], as offsets o
        // inside the span relative to 4g (the accumulator layout), lo <= o <= lo + span
        int lo = max(0, qi - w) - (ks0 + 4 * g);
        int hi = min(L - 1, qi + w) - (ks0 + 4 * g);
        const bool any = hi >= lo;
        const uint32_t span = any ? (uint32_t)(hi - lo) : 0u;
        if (!any) lo = 1 << 20;
        auto valid = [&](int kb, int i) __attribute__((always_inline)) {
            const int o = kb * 32 + (i >> 2) * 8 + (i & 3);
            return (uint32_t)(o - lo) <= span;
        };

        // exact maximum over this wave's share of the span, then P = 2^(s c - m) in fp16
        mx = NEG_INF;
#pragma unroll
        for (int j = 0; j < NKBW; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, valid(kb0 + j, i) ? s[j][i] : NEG_INF);
        mx = pair_max(mx);
        const float nb = (mx == NEG_INF) ? 0.0f : -(mx * c);

        // P of each 32-key block, its FP32 row sums, and O^T += V^T P^T right away
        o[0] = f32x16{};
        o[1] = f32x16{};
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < NKBW; ++j) {
            const int kb = kb0 + j;
            float e[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float t = __builtin_fmaf(s[j][i], c, nb);
                e[i] = __builtin_amdgcn_exp2f(valid(kb, i) ? t : NEG_INF);
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                u32x4 pk;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const f16x2 h = {(_Float16)e[8 * tt + 2 * jj], (_Float16)e[8 * tt + 2 * jj + 1]};
                    pk[jj] = __builtin_bit_cast(uint32_t, h);
                    // partial sums by block parity and half (summed in a fixed order below)
                    acc[(j & 1) * 2 + tt] = __builtin_amdgcn_fdot2(h, f16x2{(_Float16)1.0f, (_Float16)1.0f},
                                                                   acc[(j & 1) * 2 + tt], false);
                }
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    const u32x4 va = lds16(Vt + vt_off(db * 32 + r, kb * 32 + 16 * tt + 8 * g));
                    o[db] = mfma_pv(va, pk, o[db]);
                }
            }
        }
        // acc[0..1] hold the span's even blocks (block kb0 + j goes to parity j & 1)
        const bool odd = !NKF && (kb0 & 1);
        const float e0 = odd ? acc[2] : acc[0], e1 = odd ? acc[3] : acc[1];
        const float o0 = odd ? acc[0] : acc[2], o1 = odd ? acc[1] : acc[3];
        l = pair_sum((e0 + e1) + (o0 + o1));
    };
    compute(std::false_type{});

    // ---- range guard of the bf16 -> fp16 V conversion (see attn_common.hpp) ----------
    int vshift = 0;
    if constexpr (IO == IO_BF16) {
        if (wg_any<NT / 64>(!acc_finite(o, l), guard)) {
            // largest finite |v| over the staged span [ks0, ks0 + NK)
            uint32_t vmax = 0;
            for (int c = tid; c < NK * 8; c += NT) {
                const int row = ks0 + (c >> 3);
                if (row >= 0) vmax = max(vmax, bf16_finite_absmax(bload(rv, (uint32_t)row * vrb + (uint32_t)(c & 7) * 16)));
            }
            vshift = vshift_of(wg_max<NT / 64>(vmax, guard + NT / 64));
            if (vshift > 0) {
                vsc = exp2i(-vshift);
                __syncthreads();   // every wave is done with the staged span
                compute(std::true_type{});
            }
        }
    }

    if constexpr (KSPLIT > 1) {
        // Merge the shares of the query block: O = sum_v 2^(b_v - B) O_v and l likewise,
        // b_v = m_v c the base of share v (log2 units, -inf for a share with no valid key)
        // and B the largest b_v, summed in share order. Every wave writes its share to LDS
        // in rows of 64 floats (one per lane; wave w: O element e in row w * 34 + e, b in
        // row w * 34 + 32, l in row w * 34 + 33; the shares of query block wq are waves
        // wq * KSPLIT + v), then wave kq of the block merges, normalises and stores the O
        // elements E kq .. E kq + E - 1 of its lanes (E = 32 / KSPLIT), so the waves
        // share the merge and the stores.
        static_assert(WPB * KSPLIT == NT / 64 && 32 % (4 * KSPLIT) == 0, "one share per wave");
        constexpr int E = 32 / KSPLIT;           // O elements a wave merges and stores
        constexpr int SR = 34;                   // rows of 64 floats per share
        float *pb = reinterpret_cast<float *>(smem);
        const float base = (mx == NEG_INF) ? NEG_INF : mx * c;
        const int s0 = (WPB == 1 ? 0 : wq) * KSPLIT;   // the query block's first share
        __syncthreads();   // every wave is done with the staged span
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) pb[(wave * SR + db * 16 + i) * 64 + lane] = o[db][i];
        pb[(wave * SR + 32) * 64 + lane] = base;
        pb[(wave * SR + 33) * 64 + lane] = l;
        __syncthreads();
        float bv[KSPLIT];
#pragma unroll
        for (int v = 0; v < KSPLIT; ++v) bv[v] = pb[((s0 + v) * SR + 32) * 64 + lane];
        float bmax = bv[0];
#pragma unroll
        for (int v = 1; v < KSPLIT; ++v) bmax = fmaxf(bmax, bv[v]);
        // rows past L have no valid key in any share (bmax = -inf); they are not stored
        float om[E];
        {
            const float w0 = __builtin_amdgcn_exp2f(bv[0] - bmax);
            l = pb[(s0 * SR + 33) * 64 + lane] * w0;
#pragma unroll
            for (int j = 0; j < E; ++j) om[j] = pb[(s0 * SR + E * kq + j) * 64 + lane] * w0;
        }
#pragma unroll
        for (int v = 1; v < KSPLIT; ++v) {
            const float wv = __builtin_amdgcn_exp2f(bv[v] - bmax);
            l = __builtin_fmaf(wv, pb[((s0 + v) * SR + 33) * 64 + lane], l);
#pragma unroll
            for (int j = 0; j < E; ++j) om[j] = __builtin_fmaf(wv, pb[((s0 + v) * SR + E * kq + j) * 64 + lane], om[j]);
        }
        if (qi >= L) return;
        // (2^vshift undoes the guard's scaling of V; l >= 1, so inv * 2^vshift stays finite)
        const float inv = (1.0f / l) * exp2i(vshift);
        const long long row = CONTIG ? slab + (long long)qi * HD : bb * P.ob + hh * P.oh + (long long)qi * P.ol;
#pragma unroll
        for (int gg = 0; gg < E / 4; ++gg) {
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = om[gg * 4 + j] * inv;
            // accumulator elements e0 .. e0 + 3 (e0 = E kq + 4 gg): d block e0 / 16, group (e0 % 16) / 4
            const int e0 = E * kq + 4 * gg;
            const int d = (e0 >> 4) * 32 + ((e0 & 15) >> 2) * 8 + g * 4;
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
        return;
    }

    // ---- epilogue: normalise, subtract, cast, store rows < L -------------------------
    // (2^vshift undoes the guard's scaling of V; l >= 1, so inv * 2^vshift stays finite)
    const float inv = (1.0f / l) * exp2i(vshift);
    if constexpr (DIFF) {
        float *xb = reinterpret_cast<float *>(smem);
        __syncthreads();   // every wave is done with the staged span
        if (wbr == 1) {
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) xb[(wq * 32 + db * 16 + i) * 64 + lane] = o[db][i] * inv;
        }
        __syncthreads();
        if (wbr == 1) return;
    }
    if (qi >= L) return;
    const long long row = CONTIG ? slab + (long long)qi * HD : bb * P.ob + hh * P.oh + (long long)qi * P.ol;
    const float *xb = reinterpret_cast<const float *>(smem);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                y[j] = o[db][grp * 4 + j] * inv;
                if constexpr (DIFF) y[j] = y[j] - P.lam * xb[(wq * 32 + db * 16 + grp * 4 + j) * 64 + lane];
            }
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

template <int IO, bool DIFF, int NKF, bool CONTIG>
hipError_t launch_n(const LaunchArgs &a) {
    using S = NarrowShape<DIFF, NKF>;
    Params P = make_params(a);
    // short-sequence mode: every key of [0, L) is staged, so a window only masks
    P.window = (NKF && a.window < 0) ? a.L : a.window;
    P.n_qtiles = (a.L + S::BM - 1) / S::BM;
    const unsigned grid = (unsigned)P.n_qtiles * (unsigned)a.B * (unsigned)a.H;
    hipLaunchKernelGGL((attn_narrow_kernel<IO, DIFF, NKF, CONTIG>), dim3(grid), dim3(S::NT), 0,
                       static_cast<hipStream_t>(a.stream), P);
    return hipGetLastError();
}

template <int NKF, bool CONTIG>
hipError_t launch_nkc(const LaunchArgs &a) {
    const bool bf = a.dtype == 1;
    if (a.diff) return bf ? launch_n<IO_BF16, true, NKF, CONTIG>(a) : launch_n<IO_F16, true, NKF, CONTIG>(a);
    return bf ? launch_n<IO_BF16, false, NKF, CONTIG>(a) : launch_n<IO_F16, false, NKF, CONTIG>(a);
}
template <int NKF>
hipError_t launch_nk(const LaunchArgs &a) {
    return a.contig ? launch_nkc<NKF, true>(a) : launch_nkc<NKF, false>(a);
}

// Short-sequence mode for L <= 256 (span of 64, 128 or 256 keys), else windowed mode.
int span_keys(const LaunchArgs &a) { return a.L <= 64 ? 64 : a.L <= 128 ? 128 : a.L <= 256 ? 256 : 0; }

}  // namespace

bool narrow_applies(const LaunchArgs &a) { return span_keys(a) > 0 || (a.window >= 0 && a.window <= 32); }

template <int NKF>
int rows_of(const LaunchArgs &a) { return a.diff ? NarrowShape<true, NKF>::BM : NarrowShape<false, NKF>::BM; }

int narrow_tile_rows(const LaunchArgs &a) {
    switch (span_keys(a)) {
        case 64: return rows_of<64>(a);
        case 128: return rows_of<128>(a);
        case 256: return rows_of<256>(a);
        default: return rows_of<0>(a);
    }
}

int launch_narrow(const LaunchArgs &a) {
    switch (span_keys(a)) {
        case 64: return (int)launch_nk<64>(a);
        case 128: return (int)launch_nk<128>(a);
        case 256: return (int)launch_nk<256>(a);
        default: return (int)launch_nk<0>(a);
    }
}

}  // namespace sa3
