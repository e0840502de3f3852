// Pre-pass of the long-span attention kernel on gfx950: RoPE of K and the fp16 V^T
// tiles, computed once per 64-key tile into a caller-provided workspace.
//
// In the fused path every query tile that visits a key tile rotates its K rows again
// (RoPE in FP32, rounded back to the 16-bit type: "Fixes the medium DiT's FP16-mixed
// ONNX so the attention core runs FP16" discussion, section "The fix") and converts
// and transposes its V rows into the P.V operand layout; at L = 4096 that
// is 16 (plain) or 32 (differential) times per key. This pass does both once and
// writes the results in exactly the layout the long-span kernel's LDS stages hold, so
// its staging becomes a plain copy. The arithmetic is the same functions on the same
// values (rope8 / rope8_general, the same RNE casts), so the outputs of the two paths
// are bitwise identical.
//
// Workspace layout (Lp = L rounded up to 64; rows and keys in [L, Lp) are zero):
//   K' [branch][B*H][Lp][D]  rotated K rows, IO type;
//   V' [B*H][Lp/64][D][64]   fp16; per tile, row d holds the 64 keys' values of dim d
//                            with bits 2 and 3 of the key index swapped (the order in
//                            which one lane's P.V operand is 8 consecutive keys).
// One workgroup of 256 threads per (b, h, key tile); memory-bound: it reads K (each
// branch), V and the table rows once and writes K' and V' once.

#include "attn_common.hpp"

namespace sa3 {
namespace {

template <int IO, bool DIFF, bool CONTIG, int D>
__global__ __launch_bounds__(256) void attn_prep_kernel(Params P) {
    constexpr int NT = 256;
    constexpr int NBS = DIFF ? 2 : 1;
    constexpr int RB = D * 2;                // bytes per row of q/k/v and of the default table
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int KC = BN * CPR / NT;        // K chunks per thread per branch
    constexpr int VD = BN * D / (2 * NT);    // d values per thread for its two keys
    constexpr int NV = VD / 8;               // 16-byte V loads per key
    constexpr int VC = D * BN / (8 * NT);    // 16-byte V' chunks per thread
    static_assert(KC >= 1 && NV >= 1 && VC >= 1, "head dim 64 or 128");
    __shared__ __attribute__((aligned(16))) uint16_t vt[D * VT_STRIDE];

    const int tid = threadIdx.x;
    const int ntiles = P.ws_tiles;
    // the split tail's counters (long-span kernel) start each call at zero
    if (blockIdx.x == 0)
        for (int i = tid; i < P.n_tail; i += NT) P.cnt[i] = 0u;
    const int bh = blockIdx.x / ntiles;
    const int t = blockIdx.x - bh * ntiles;
    const int bb = bh / P.H, hh = bh - bb * P.H;
    const int BH = gridDim.x / ntiles;
    const int L = P.L;
    const long long lp = (long long)ntiles * BN;
    const uint32_t krb = CONTIG ? (uint32_t)RB : P.k_rowb;
    const uint32_t vrb = CONTIG ? (uint32_t)RB : P.v_rowb;
    const long long slab = (long long)bh * L * D;
    const long long kbr = CONTIG ? (long long)BH * L * D : P.k_br;
    const uint32_t trb = CONTIG ? (uint32_t)RB : P.tab_rowb;
    const rsrc_t rc = make_rsrc(P.cos, (uint32_t)L * trb);
    const rsrc_t rs = make_rsrc(P.sin, (uint32_t)L * trb);
    constexpr uint32_t NOWHERE = 0xfffffff0u;   // an offset past every buffer: reads zeros

    // ---- K: chunk c = tid + i * NT is row c / CPR, dims 8 (c % CPR) .. +7 ------------
    const int cc = tid % CPR;
    const RopeChunk kch = rope_chunk(cc, P.rope_half, P.rot_dim);
#pragma unroll
    for (int br = 0; br < NBS; ++br) {
        const rsrc_t rk = slab_rsrc(P.k, br * kbr + (CONTIG ? slab : bb * P.kb + hh * P.kh), krb, L, RB);
        uint16_t *dst = P.kw + ((long long)br * BH + bh) * lp * D;
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const uint32_t row = (uint32_t)(t * BN + tid / CPR + i * (NT / CPR));
            u32x4 rot;
            if constexpr (CONTIG) {
                const uint32_t off = row * RB + (uint32_t)cc * 16;
                rot = rope8<IO>(bload(rk, off), bload(rc, off), bload(rs, off));
            } else {
                const uint32_t to = kch.mode ? row * trb + kch.toff : NOWHERE;
                const uint32_t t1 = kch.mode >= 2 ? to + 16 : NOWHERE;
                const uint32_t po = kch.mode >= 2 ? row * krb + (uint32_t)kch.partner * 16 : NOWHERE;
                rot = rope8_general<IO>(bload(rk, row * krb + (uint32_t)cc * 16), bload(rk, po), bload(rc, to),
                                        bload(rc, t1), bload(rs, to), bload(rs, t1), kch.mode);
            }
            *reinterpret_cast<u32x4 *>(dst + (long long)row * D + cc * 8) = rot;
        }
    }

    // ---- V: keys 2p, 2p+1 (p = tid % 32), VD dims from VD * (tid / 32) -----------------
    const rsrc_t rv = slab_rsrc(P.v, CONTIG ? slab : bb * P.vb + hh * P.vh, vrb, L, RB);
    const int vp = tid & 31;
    const int vd0 = (tid >> 5) * VD;
    const uint32_t r0 = (uint32_t)(t * BN + 2 * vp);
    u32x4 raw[2][NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        raw[0][n] = bload(rv, r0 * vrb + (uint32_t)vd0 * 2 + 16 * n);
        raw[1][n] = bload(rv, (r0 + 1) * vrb + (uint32_t)vd0 * 2 + 16 * n);
    }
    const int vpos = (2 * vp & ~12) | ((2 * vp & 4) << 1) | ((2 * vp & 8) >> 1);
#pragma unroll
    for (int j = 0; j < VD; ++j) {
        const uint32_t wa = raw[0][j >> 3][(j >> 1) & 3], wb = raw[1][j >> 3][(j >> 1) & 3];
        uint32_t w;
        if constexpr (IO == IO_BF16) {
            const float fa = __uint_as_float((j & 1) ? (wa & 0xffff0000u) : (wa << 16));
            const float fb = __uint_as_float((j & 1) ? (wb & 0xffff0000u) : (wb << 16));
            w = pack2<IO_F16>(fa, fb);
        } else {
            w = (j & 1) ? __builtin_amdgcn_perm(wb, wa, 0x07060302u) : __builtin_amdgcn_perm(wb, wa, 0x05040100u);
        }
        *reinterpret_cast<uint32_t *>(vt + (vd0 + j) * VT_STRIDE + vpos) = w;
    }
    __syncthreads();
    // V' tile: D rows of 64 keys, 8 chunks of 16 bytes per row
    uint16_t *vdst = P.vw + ((long long)bh * ntiles + t) * D * BN;
#pragma unroll
    for (int i = 0; i < VC; ++i) {
        const int c = tid + i * NT;
        const int d = c >> 3, kc = c & 7;
        *reinterpret_cast<u32x4 *>(vdst + d * BN + kc * 8) =
            *reinterpret_cast<const u32x4 *>(vt + d * VT_STRIDE + kc * 8);
    }
}

template <int IO, bool DIFF, bool CONTIG, int D>
hipError_t launch(const LaunchArgs &a) {
    Params P = make_params(a);
    set_tail(P, a);   // its counters are cleared here
    const unsigned grid = (unsigned)P.ws_tiles * (unsigned)a.B * (unsigned)a.H;
    hipLaunchKernelGGL((attn_prep_kernel<IO, DIFF, CONTIG, D>), dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(a.stream), P);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const LaunchArgs &a) {
    const bool bf = a.dtype == 1;
    if (a.contig) {
        if (a.diff) return bf ? launch<IO_BF16, true, true, D>(a) : launch<IO_F16, true, true, D>(a);
        return bf ? launch<IO_BF16, false, true, D>(a) : launch<IO_F16, false, true, D>(a);
    }
    if (a.diff) return bf ? launch<IO_BF16, true, false, D>(a) : launch<IO_F16, true, false, D>(a);
    return bf ? launch<IO_BF16, false, false, D>(a) : launch<IO_F16, false, false, D>(a);
}

}  // namespace

int launch_prep(const LaunchArgs &a) {
    return (int)(a.D == 128 ? launch_d<128>(a) : launch_d<64>(a));
}

}  // namespace sa3
