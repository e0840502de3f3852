/*
 * sa3attn.h -- C ABI of the fused RoPE attention core for AMD MI355X (gfx950).
 *
 * The operation is the attention core of the Stable Audio 3 transformers:
 *
 *   q' = cast_io(RoPE_fp32(q)),  k' = cast_io(RoPE_fp32(k))
 *   out = softmax(scale * q' k'^T + M) v                        (plain)
 *   out = softmax(scale * q1' k1'^T + M) v
 *         - lambda * softmax(scale * q2' k2'^T + M) v           (differential)
 *
 * Sources (the pages describing the method):
 *  - RoPE is computed in FP32 and cast back to the activation dtype before QK^T;
 *    attention then runs on FP16 inputs with the softmax accumulated in FP32
 *    inside the fused kernel ("Fixes the medium DiT's FP16-mixed ONNX so the
 *    attention core runs FP16" discussion, sections "The bug" and "The fix").
 *  - The cos/sin table is computed on the host in FP32 and frozen as a constant,
 *    sized to a maximum length (sa3_trt README, section "DiT precision").
 *  - M is a sliding window of half-width w, "+-WINDOW" around each query
 *    (Stable Audio 3 TensorRT engines README, section "Building your own").
 *  - The differential variant shares V between two softmax branches; the two
 *    branch results are subtracted after accumulation, in FP32 (same README,
 *    section "How the kernels differ").
 *  - The forward must be capturable into a stream graph with no host callbacks
 *    (same README, section "Why JIT breaks on sm_120").
 *
 * Conventions shared by every entry point
 *  - Layout: every tensor is row-major contiguous [B][H][L][D], D fastest.
 *    Differential q and k are stacked [2][B][H][L][D] (branch 1, then branch 2);
 *    v is [B][H][L][D] and shared by both branches. sa3attn_forward_strided takes
 *    the same tensors with explicit strides instead (below).
 *  - Every device pointer (q, k, v, cos, sin, out) is 16-byte aligned.
 *  - RoPE rotates adjacent pairs (x[2i], x[2i+1]) at position m = 0..L-1 of each
 *    (b, h) slab: r0 = fl(fl(x0 c) - fl(x1 s)), r1 = fl(fl(x0 s) + fl(x1 c)) in FP32,
 *    then rounds to nearest-even to the IO dtype.
 *  - cos, sin: FP32 tables [L_tab][D/2] ([L_tab][R/2] with a partial rotary width
 *    R, see sa3attn_forward_general), L_tab >= L; row m holds cos(m theta_i) and
 *    sin(m theta_i), shared across B and H. Only rows < L are read. The library
 *    cannot check L_tab: passing a shorter table is a caller error.
 *  - window: half-width w; key j is masked for query i when |i - j| > w.
 *    window < 0 means full attention. There is no causal mask.
 *  - scale multiplies the FP32 QK^T accumulator (not folded into q).
 *  - Ownership: the caller allocates and owns every buffer (device memory for
 *    q, k, v, cos, sin, out, and the workspace of sa3attn_forward_ws). The library
 *    never allocates, frees or synchronises and keeps no pointer after returning.
 *    Work (one kernel; two with the pre-pass of sa3attn_forward_ws) is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) and can be captured into a
 *    graph.
 *  - out must not overlap any input.
 *  - Errors: validation runs before any launch; on error nothing is enqueued and
 *    `out` is untouched. Status codes are below; sa3attn_status_string() names them.
 *  - Thread safety: calls may be made from several threads; the only shared state
 *    is a per-device capability cache filled once.
 *  - Supported: D = 64 or 128, IO dtype fp16 or bf16, out dtype fp16, bf16 or
 *    fp32, 1 <= L <= 2^30 / D (16777216 at D = 64), and grid size
 *    (ceil(L/tile) * B * H) below 2^31.
 *  - Numerics: QK^T and P.V run on MFMA with FP32 accumulation; the running
 *    softmax max and sum are FP32. P is rounded to fp16 before P.V for both IO
 *    dtypes; with bf16 inputs V is converted to fp16 as it is staged, which is
 *    exact for |v| in [2^-14, 65504]. A bf16 V beyond fp16's range (|v| >= 65536,
 *    up to bf16's largest finite value) is handled on the device: a workgroup whose
 *    accumulators come out non-finite finds the largest finite |v| of the keys it
 *    visited and redoes its work with V scaled by an exact power of two, undone in
 *    the output (so large finite V gives finite, accurate results; that workgroup
 *    takes about twice as long). Non-finite inputs give non-finite outputs.
 */
#ifndef SA3ATTN_H
#define SA3ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

#define SA3ATTN_VERSION_MAJOR 0
#define SA3ATTN_VERSION_MINOR 6

/* Status codes. */
enum {
    SA3_OK = 0,
    SA3_ERR_NULL = -1,         /* a required pointer is NULL                          */
    SA3_ERR_SHAPE = -2,        /* B, H, L or D < 1, D odd, or a size overflows        */
    SA3_ERR_UNSUPPORTED = -3,  /* D not 64 or 128, or an unknown dtype                 */
    SA3_ERR_ARG = -4,          /* non-finite scale or lambda, out overlaps an input,
                                  a misaligned pointer, or unusable strides           */
    SA3_ERR_DEVICE = -5,       /* no HIP device, or the current device is not gfx950  */
    SA3_ERR_LAUNCH = -6,       /* the kernel launch failed (hipGetLastError)          */
    SA3_ERR_SCRATCH = -7       /* sa3attn_forward_noalloc: the pre-pass workspace the
                                  policy asks for exceeds SA3ATTN_SCRATCH_BYTES        */
};

/* Element types. */
enum { SA3_F16 = 0, SA3_BF16 = 1, SA3_F32 = 2 };

/*
 * sa3attn_forward -- fp16 q/k/v in, fp16 out.
 * Differential exactly when lambda != 0; then q and k point to stacked
 * [2][B][H][L][D] buffers. Returns a status code.
 */
int sa3attn_forward(const void *q, const void *k, const void *v,
                    const float *cos, const float *sin, void *out,
                    int B, int H, int L, int D,
                    int window, float lambda, float scale, void *stream);

/* sa3attn_forward_bf16 -- the same arguments and rules, bf16 in and bf16 out. */
int sa3attn_forward_bf16(const void *q, const void *k, const void *v,
                         const float *cos, const float *sin, void *out,
                         int B, int H, int L, int D,
                         int window, float lambda, float scale, void *stream);

/*
 * sa3attn_desc / sa3attn_forward_ex -- the explicit form.
 *   dtype:        SA3_F16 or SA3_BF16 (q, k, v)
 *   out_dtype:    SA3_F16, SA3_BF16 or SA3_F32
 *   differential: 0 = plain; 1 = two branches (q, k stacked), independent of
 *                 lambda, so lambda = 0 still runs both branches.
 * Other fields as in sa3attn_forward.
 */
typedef struct sa3attn_desc {
    const void *q;
    const void *k;
    const void *v;
    const float *cos;
    const float *sin;
    void *out;
    int B, H, L, D;
    int window;
    float lambda;
    float scale;
    int dtype;
    int out_dtype;
    int differential;
    void *stream;
} sa3attn_desc;

int sa3attn_forward_ex(const sa3attn_desc *desc);

/*
 * sa3attn_strides / sa3attn_forward_strided -- the explicit form over strided views.
 * Element (b, h, l, d) of q is at q + q[0]*b + q[1]*h + q[2]*l + d (in elements of
 * the tensor's own type; the head dim is contiguous), and likewise for k, v and out.
 * Differential branch 2 of q (of k) starts q_branch (k_branch) elements after
 * branch 1. The layout a fused QKV projection writes, [B][L][H][D], is
 * {L*H*D, D, H*D}; sa3attn_forward_ex is this call with contiguous [B][H][L][D]
 * strides {H*L*D, L*D, D} and branch strides B*H*L*D.
 * Requirements (SA3_ERR_ARG otherwise, before anything is enqueued): every stride
 * >= 0 and a multiple of 8 elements; the l stride >= D; (L + 128) * l stride * 2
 * < 2^32 for q, k, v and out; the output view gives every (b, h, l) its own row;
 * out overlaps no input. Inputs may alias each other (they are only read).
 * A NULL strides pointer returns SA3_ERR_NULL. The strides are copied; the
 * caller keeps ownership of the struct.
 */
typedef struct sa3attn_strides {
    long long q[3];
    long long k[3];
    long long v[3];
    long long out[3];
    long long q_branch;
    long long k_branch;
} sa3attn_strides;

int sa3attn_forward_strided(const sa3attn_desc *desc, const sa3attn_strides *strides);

/*
 * sa3attn_rope / sa3attn_forward_general -- RoPE options and the most general form.
 * The pages do not pin which dims RoPE pairs up; the default (every other entry
 * point) is adjacent pairs over the whole head dim. Options:
 *   pairing:    SA3_ROPE_ADJACENT, pairs (x[2i], x[2i+1]), or SA3_ROPE_HALF, pairs
 *               (x[i], x[i + R/2]) (the rotate-half convention), i = 0 .. R/2 - 1;
 *   rotary_dim: R, the leading dims rotated: a multiple of 16, 16 <= R <= D; dims
 *               R .. D-1 pass through unchanged.
 * Pair i uses table column i: cos and sin are then [L_tab][R/2] (sa3attn_rope_table
 * with D = R gives theta_i = base^(-2i/R)). The FP32 arithmetic per pair and the
 * cast back are the same as for the default.
 * strides NULL = contiguous [B][H][L][D] (as sa3attn_forward_ex); rope NULL =
 * the default. Bad options return SA3_ERR_ARG before anything is enqueued.
 */
enum { SA3_ROPE_ADJACENT = 0, SA3_ROPE_HALF = 1 };
typedef struct sa3attn_rope {
    int pairing;
    int rotary_dim;
} sa3attn_rope;

int sa3attn_forward_general(const sa3attn_desc *desc, const sa3attn_strides *strides,
                            const sa3attn_rope *rope);

/*
 * sa3attn_workspace_bytes / sa3attn_forward_ws -- the general form with a pre-pass.
 * The RoPE of a key row (rotate in FP32, round back; the FP16-fix discussion of the
 * medium DiT's ONNX, section "The fix") does not depend on the query, yet
 * the fused kernel redoes it, and the fp16 transposition of V, for every query tile
 * that visits the key: 16 to 32 times per key at L = 4096. With a workspace the
 * library first runs a pre-pass kernel that rotates K (each branch) and converts and
 * transposes V once, into the workspace, and the attention kernel then copies its
 * key tiles from there. Outputs are bitwise identical to sa3attn_forward_general's for
 *     differential calls, persistent grids and D = 128 without a split tail; plain D = 64
 *     calls of one round per query tile walk the keys 128 at a time with the pre-pass
 *     (one softmax base move per 128 keys instead of 64), and the two kinds of grid
 *     below take the keys in other groups: there the sums over a row's keys are taken
 *     in another order (the same bar against the exact result, other last bits; calls
 *     of the same shape and policy give the same bits run to run).
 *   Small grids: plain calls (not differential) at D = 64 outside the single-span
 *     kernel whose 256-row query tiles number fewer than the device's compute units
 *     (B x H x ceil(L / 256) < CUs) and whose 64-row tiles fit two per compute unit
 *     (B x H x ceil(L / 64) <= 2 x CUs). With the pre-pass they run 64-row tiles:
 *     full attention on contiguous tensors with the default RoPE in a key-split kernel
 *     (each tile's keys in two halves on separate waves, merged at the end), other
 *     calls in 2-wave workgroups of the long-span kernel (the same bits).
 *   Split tail: other long-span calls whose grid of query tiles (256 rows, 128
 *     differential; T = B x H x ceil(L / rows)) leaves a last round of r = T mod CUs
 *     tiles with 0 < r <= CUs / 2, except grids of more tiles than CUs whose tiles span
 *     at most 32 key tiles (which run persistent when contiguous). With the pre-pass
 *     each of those r tiles is split into k = min(4, CUs / r) contiguous key ranges of
 *     at least 4 key tiles (k >= 2), one workgroup each; the last range to finish a
 *     tile merges the ranges' partial results, which the workspace holds after K' and
 *     V' (r x k x 8 x 64 x (D / 32 x 16 + 4) floats, then r counters in 256-byte units).
 *   policy: SA3_PREP_AUTO runs the pre-pass on small grids and split-tail grids, and
 *     otherwise when a key tile is visited by enough query tiles (query tiles of 256
 *     rows plain, 128 differential; full attention: ceil(L / rows) visits; a window of
 *     half-width w: about (2w + 64) / rows + 1): at least 3 at D = 128; at D = 64 at
 *     least 10 plain or 18 differential, except on grids of more tiles than compute
 *     units whose tiles span at most 32 key tiles (contiguous calls there run
 *     persistent): at least 9 differential there, and 12 plain for contiguous calls
 *     (256 compute units are assumed when no device is current); the shapes where it
 *     measured faster. SA3_PREP_ALWAYS whenever the call
 *     takes the long-span kernel; SA3_PREP_NEVER never. SA3_PREP_ONLY enqueues the
 *     pre-pass alone (out is not written) and SA3_PREP_REUSE the attention kernel
 *     alone, reading a workspace that an earlier ALWAYS or ONLY call filled from the
 *     same k, v, cos, sin, shape, strides and RoPE options (so K and V prepared once
 *     serve several q; the library cannot check the contents: stale ones give wrong
 *     outputs, never out-of-bounds accesses). Calls that take the single-span kernel
 *     (windows of half-width <= 32, or L <= 256, at D = 64) have no pre-pass under
 *     any policy: ONLY then enqueues nothing and REUSE runs the call as usual.
 *   sa3attn_workspace_bytes: *bytes = the workspace the call shape takes under
 *     `policy`: (2 or 3, differential) x B x H x ceil(L/64)*64 x D x 2 bytes when
 *     the pre-pass runs, plus the split tail's partials and counters where it
 *     applies, else 0 (the compute-unit count is the current device's). Reads only
 *     B, H, L, D, window, dtype, out_dtype and differential of desc; shape errors as
 *     sa3attn_forward_ex's, SA3_ERR_NULL for a NULL desc or bytes, SA3_ERR_ARG for an
 *     unknown policy.
 *   sa3attn_forward_ws: sa3attn_forward_general plus
 *     workspace: device memory of workspace_bytes bytes (at least what
 *       sa3attn_workspace_bytes gives for the same shape and policy), 16-byte
 *       aligned, overlapping no input and not out; owned by the caller; its contents
 *       on entry do not matter and on return are scratch. Calls that may run
 *       concurrently need workspaces of their own. May be NULL when the size is 0.
 *   When the pre-pass runs, a NULL workspace returns SA3_ERR_NULL and a smaller,
 *   misaligned or overlapping one SA3_ERR_ARG; an unknown policy is SA3_ERR_ARG;
 *   all before anything is enqueued. With the pre-pass, two kernels are enqueued on
 *   the stream, in order.
 */
enum { SA3_PREP_AUTO = 0, SA3_PREP_ALWAYS = 1, SA3_PREP_NEVER = 2, SA3_PREP_ONLY = 3, SA3_PREP_REUSE = 4 };

int sa3attn_workspace_bytes(const sa3attn_desc *desc, int policy, unsigned long long *bytes);
int sa3attn_forward_ws(const sa3attn_desc *desc, const sa3attn_strides *strides,
                       const sa3attn_rope *rope, void *workspace,
                       unsigned long long workspace_bytes, int policy);

/*
 * sa3attn_forward_noalloc -- sa3attn_forward_ws without a caller workspace, for
 * callers that cannot allocate device memory (code under graph capture, serving
 * loops or harnesses that forbid allocation): the pre-pass workspace is a static
 * device array of the library, SA3ATTN_SCRATCH_BYTES (64 MiB) on each GPU the
 * library runs on, held until the process ends. The call itself allocates nothing;
 * its first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress) and caches it.
 *   desc, strides, rope: as for sa3attn_forward_general; the caller still provides
 *     q, k, v, cos, sin and out.
 *   policy: as for sa3attn_forward_ws. When the pre-pass with the split tail's
 *     partials would need more than SA3ATTN_SCRATCH_BYTES (sa3attn_workspace_bytes
 *     gives the size) but K' and V' alone fit, the call runs the pre-pass without the
 *     split tail (its last round whole: other last bits than the workspace call's, the
 *     same bar). When K' and V' alone do not fit either: AUTO runs the call without the
 *     pre-pass (bitwise as NEVER); ALWAYS, ONLY and REUSE return SA3_ERR_SCRATCH before
 *     anything is enqueued.
 *   Sharing: every call on one GPU uses the same array, whose contents persist from
 *     call to call (REUSE reads what the last ALWAYS or ONLY call on that GPU wrote).
 *     Calls that may overlap in time on one GPU (other streams, other threads) race
 *     on it and give wrong outputs; order them, or use sa3attn_forward_ws with a
 *     workspace per stream. Nothing in the array needs to start at zero.
 *   Errors as for sa3attn_forward_ws, plus SA3_ERR_SCRATCH, and SA3_ERR_DEVICE when
 *   the array's address cannot be looked up.
 */
#define SA3ATTN_SCRATCH_BYTES (64ull << 20)

int sa3attn_forward_noalloc(const sa3attn_desc *desc, const sa3attn_strides *strides,
                            const sa3attn_rope *rope, int policy);

/*
 * sa3attn_rope_table -- fill a host FP32 cos/sin table [L][D/2].
 * theta_i = base^(-2i/D) (the double nearest the real value, from an
 * extended-precision power); entry [m][i] = fp32(cos(m * theta_i)) and
 * fp32(sin(m * theta_i)), each one rounding of the fp64 value (sa3_trt README,
 * section "DiT precision": host-computed FP32 table). cos and sin are host
 * pointers to L*D/2 floats owned by the caller. Returns SA3_OK, SA3_ERR_NULL,
 * SA3_ERR_SHAPE (L < 1, D < 2 or odd) or SA3_ERR_ARG (base not finite and > 0).
 */
int sa3attn_rope_table(float *cos, float *sin, int L, int D, double base);

/* sa3attn_status_string -- a static, human-readable name for a status code. */
const char *sa3attn_status_string(int status);

/* sa3attn_version -- (major << 16) | minor of the library that is loaded. */
int sa3attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SA3ATTN_H */
