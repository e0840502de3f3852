// C-ABI entry points of the fused RoPE attention core (declared in include/sa3attn.h):
// argument validation, device capability check, dispatch to the gfx950 kernels.
//
// Validation happens before anything touches the GPU so that a bad call enqueues
// nothing and leaves `out` untouched; a failure is never reported as zeros (the
// Stable Audio 3 TensorRT engines README, section "Building your own", lists
// silent-zero and wrong-argument-order failures of the kernels it describes).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "sa3attn.h"
#include "sa3attn_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxL = 1 << 24;
// 0 = not checked yet, 1 = gfx950, 2 = something else
std::atomic<int> g_dev_ok[kMaxDevices];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return SA3_ERR_DEVICE;
    }
    if (dev >= kMaxDevices) return SA3_ERR_DEVICE;
    int s = g_dev_ok[dev].load(std::memory_order_acquire);
    if (s == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return SA3_ERR_DEVICE;
        }
        s = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_ok[dev].store(s, std::memory_order_release);
    }
    return s == 1 ? SA3_OK : SA3_ERR_DEVICE;
}

// Compute units of the current device, cached per device; 256 (an MI355X) when there is
// no usable device, so that host-only queries answer the same as calls on that part.
constexpr int kDefaultCUs = 256;
std::atomic<int> g_dev_cus[kMaxDevices];

int device_cus() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kDefaultCUs;
    }
    int n = g_dev_cus[dev].load(std::memory_order_acquire);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            return kDefaultCUs;
        }
        g_dev_cus[dev].store(n, std::memory_order_release);
    }
    return n;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes from the first to one past the last element a [B][H][L][D] view with element
// strides s = {b, h, l} (d contiguous) can touch; non-negative strides.
unsigned long long extent_bytes(const long long s[3], int B, int H, int L, int D, int elem) {
    const unsigned long long last = (unsigned long long)(B - 1) * (unsigned long long)s[0] +
                                    (unsigned long long)(H - 1) * (unsigned long long)s[1] +
                                    (unsigned long long)(L - 1) * (unsigned long long)s[2] + (unsigned long long)D;
    return last * (unsigned long long)elem;
}

// Strides the kernels can use: non-negative, multiples of 8 elements (16-byte chunks),
// a position stride of at least one row, and 32-bit row offsets: the kernels read up
// to 64 rows past either end of a slab and rely on those offsets (negative ones wrap
// modulo 2^32) landing at or above the slab's buffer range, which then reads zeros.
bool strides_ok(const long long s[3], int L, int D) {
    for (int i = 0; i < 3; ++i)
        if (s[i] < 0 || (s[i] & 7) != 0 || s[i] > (1ll << 40)) return false;
    if (s[2] < D) return false;
    return (unsigned long long)(L + 128) * (unsigned long long)s[2] * 2ull < (1ull << 32);
}

// The output view maps every (b, h, l) row to its own D elements: with the dimensions
// of size > 1 sorted by stride, each stride is at least the span of the ones inside it.
bool rows_distinct(const long long s[3], int B, int H, int L, int D) {
    long long st[3] = {s[0], s[1], s[2]};
    long long n[3] = {B, H, L};
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (st[j] < st[i]) {
                const long long a = st[i], b = n[i];
                st[i] = st[j];
                n[i] = n[j];
                st[j] = a;
                n[j] = b;
            }
    long long span = D;
    for (int i = 0; i < 3; ++i) {
        if (n[i] == 1) continue;
        if (st[i] < span) return false;
        span = st[i] * n[i];
    }
    return true;
}

// The workspace arguments of sa3attn_forward_ws (absent for the other entry points);
// scratch: sa3attn_forward_noalloc, whose workspace is the library's static device array.
struct Workspace {
    void *ptr;
    unsigned long long bytes;
    int policy;
    bool scratch;
};

// Shape and type checks shared by every entry point.
int check_shape(const sa3attn_desc *d) {
    if (d->B < 1 || d->H < 1 || d->L < 1 || d->D < 1 || (d->D & 1)) return SA3_ERR_SHAPE;
    if (d->L > kMaxL) return SA3_ERR_SHAPE;
    if (d->D != 64 && d->D != 128) return SA3_ERR_UNSUPPORTED;
    if ((long long)d->L * d->D > (1ll << 30)) return SA3_ERR_SHAPE;   // 32-bit row offsets
    if (d->dtype != SA3_F16 && d->dtype != SA3_BF16) return SA3_ERR_UNSUPPORTED;
    if (d->out_dtype != SA3_F16 && d->out_dtype != SA3_BF16 && d->out_dtype != SA3_F32)
        return SA3_ERR_UNSUPPORTED;
    if (d->differential != 0 && d->differential != 1) return SA3_ERR_ARG;
    const unsigned long long bh = (unsigned long long)d->B * (unsigned long long)d->H;
    const unsigned long long elems = bh * (unsigned long long)d->L * (unsigned long long)d->D;
    if (bh > (1ull << 31) || elems > (1ull << 56)) return SA3_ERR_SHAPE;
    return SA3_OK;
}

// The launch fields that decide which kernel runs (and so the workspace size).
void shape_args(const sa3attn_desc *d, sa3::LaunchArgs &a) {
    a.n_cu = device_cus();
    a.tail_ok = 1;
    a.B = d->B;
    a.H = d->H;
    a.L = d->L;
    a.D = d->D;
    // a window reaching every key is full attention: |i - j| <= L - 1 always holds
    a.window = (d->window < 0 || d->window >= d->L - 1) ? -1 : d->window;
    a.dtype = d->dtype;
    a.out_dtype = d->out_dtype;
    a.diff = d->differential;
}

bool policy_ok(int p) {
    return p == SA3_PREP_AUTO || p == SA3_PREP_ALWAYS || p == SA3_PREP_NEVER || p == SA3_PREP_ONLY ||
           p == SA3_PREP_REUSE;
}

// Workspace bytes the pre-pass takes under `policy` (0: it does not run).
unsigned long long prep_need(const sa3::LaunchArgs &a, int policy) {
    if (policy == SA3_PREP_NEVER || (policy == SA3_PREP_AUTO && !sa3::prep_pays(a))) return 0;
    return sa3::prep_bytes(a);
}

int forward_impl(const sa3attn_desc *d, const sa3attn_strides *sp, const sa3attn_rope *rp,
                 const Workspace *ws = nullptr) {
    if (!d) return SA3_ERR_NULL;
    if (!d->q || !d->k || !d->v || !d->cos || !d->sin || !d->out) return SA3_ERR_NULL;
    const int shape = check_shape(d);
    if (shape != SA3_OK) return shape;
    if (!std::isfinite(d->scale) || !std::isfinite(d->lambda)) return SA3_ERR_ARG;
    if (ws && !policy_ok(ws->policy)) return SA3_ERR_ARG;

    const unsigned long long bh = (unsigned long long)d->B * (unsigned long long)d->H;
    const unsigned long long elems = bh * (unsigned long long)d->L * (unsigned long long)d->D;

    // strides: given, or those of contiguous [B][H][L][D] (q, k stacked [2][...])
    sa3attn_strides s;
    if (sp) {
        s = *sp;
    } else {
        const long long c[3] = {(long long)d->H * d->L * d->D, (long long)d->L * d->D, d->D};
        for (int i = 0; i < 3; ++i) s.q[i] = s.k[i] = s.v[i] = s.out[i] = c[i];
        s.q_branch = s.k_branch = (long long)elems;
    }
    if (!strides_ok(s.q, d->L, d->D) || !strides_ok(s.k, d->L, d->D) || !strides_ok(s.v, d->L, d->D) ||
        !strides_ok(s.out, d->L, d->D))
        return SA3_ERR_ARG;
    if (d->differential && (s.q_branch < 0 || (s.q_branch & 7) || s.k_branch < 0 || (s.k_branch & 7)))
        return SA3_ERR_ARG;
    if (!rows_distinct(s.out, d->B, d->H, d->L, d->D)) return SA3_ERR_ARG;
    // RoPE options: adjacent or half-split pairs over the leading R dims
    const int pairing = rp ? rp->pairing : SA3_ROPE_ADJACENT;
    const int rot_dim = rp ? rp->rotary_dim : d->D;
    if (pairing != SA3_ROPE_ADJACENT && pairing != SA3_ROPE_HALF) return SA3_ERR_ARG;
    if (rot_dim < 16 || rot_dim > d->D || (rot_dim & 15)) return SA3_ERR_ARG;
    if (!aligned16(d->q) || !aligned16(d->k) || !aligned16(d->v) || !aligned16(d->out) || !aligned16(d->cos) ||
        !aligned16(d->sin))
        return SA3_ERR_ARG;

    // out must not overlap any input (byte ranges the views can reach)
    const int osz = d->out_dtype == SA3_F32 ? 4 : 2;
    const size_t out_bytes = (size_t)extent_bytes(s.out, d->B, d->H, d->L, d->D, osz);
    const size_t q_bytes = (size_t)(extent_bytes(s.q, d->B, d->H, d->L, d->D, 2) +
                                    (d->differential ? (unsigned long long)s.q_branch * 2ull : 0ull));
    const size_t k_bytes = (size_t)(extent_bytes(s.k, d->B, d->H, d->L, d->D, 2) +
                                    (d->differential ? (unsigned long long)s.k_branch * 2ull : 0ull));
    const size_t v_bytes = (size_t)extent_bytes(s.v, d->B, d->H, d->L, d->D, 2);
    const size_t tab_bytes = (size_t)d->L * (size_t)(rot_dim / 2) * sizeof(float);
    if (overlaps(d->out, out_bytes, d->q, q_bytes) || overlaps(d->out, out_bytes, d->k, k_bytes) ||
        overlaps(d->out, out_bytes, d->v, v_bytes) || overlaps(d->out, out_bytes, d->cos, tab_bytes) ||
        overlaps(d->out, out_bytes, d->sin, tab_bytes))
        return SA3_ERR_ARG;

    sa3::LaunchArgs a;
    a.q = d->q;
    a.k = d->k;
    a.v = d->v;
    a.cos = d->cos;
    a.sin = d->sin;
    a.out = d->out;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = s.q[i];
        a.ks[i] = s.k[i];
        a.vs[i] = s.v[i];
        a.os[i] = s.out[i];
    }
    a.q_br = s.q_branch;
    a.k_br = s.k_branch;
    {
        const long long c[3] = {(long long)d->H * d->L * d->D, (long long)d->L * d->D, d->D};
        bool contig = true;
        for (int i = 0; i < 3; ++i)
            contig = contig && s.q[i] == c[i] && s.k[i] == c[i] && s.v[i] == c[i] && s.out[i] == c[i];
        if (d->differential) contig = contig && s.q_branch == (long long)elems && s.k_branch == (long long)elems;
        contig = contig && pairing == SA3_ROPE_ADJACENT && rot_dim == d->D;
        a.contig = contig ? 1 : 0;
    }
    a.rope_half = pairing == SA3_ROPE_HALF ? 1 : 0;
    a.rot_dim = rot_dim;
    shape_args(d, a);
    a.lam = d->lambda;
    a.scale_log2 = (float)(std::fabs((double)d->scale) * 1.4426950408889634074);
    // masked keys carry -inf scores into s * c: with scale 0 use the smallest normal
    // float instead (-inf * c stays -inf, and every finite s * c still rounds 2^(s c - m)
    // to exactly 1, the value scale 0 gives)
    if (a.scale_log2 == 0.0f) a.scale_log2 = FLT_MIN;
    a.neg_scale = d->scale < 0.0f ? 1 : 0;
    a.stream = d->stream;
    a.ws = nullptr;
    a.prep = 0;
    a.run_prep = 0;
    a.run_main = 1;
    if (!std::isfinite(a.scale_log2)) return SA3_ERR_ARG;

    // workspace of the pre-pass, when the policy runs it for this call: it must hold
    // prep_bytes, be 16-byte aligned and overlap neither an input nor out (the static
    // scratch is a separate allocation of fixed size: AUTO skips the pre-pass when the
    // scratch is too small, the other policies are an error)
    unsigned long long need = ws ? prep_need(a, ws->policy) : 0;
    if (ws && ws->scratch && need > sa3::kScratchBytes) {
        // without the split tail's partials the pre-pass may still fit
        a.tail_ok = 0;
        need = prep_need(a, ws->policy);
    }
    if (ws && ws->scratch && need > sa3::kScratchBytes) {
        if (ws->policy != SA3_PREP_AUTO) return SA3_ERR_SCRATCH;
        need = 0;
    }
    if (ws && ws->policy == SA3_PREP_ONLY) a.run_main = 0;
    if (need > 0) {
        if (!ws->scratch) {
            if (!ws->ptr) return SA3_ERR_NULL;
            if (ws->bytes < need || !aligned16(ws->ptr)) return SA3_ERR_ARG;
            const size_t wb = (size_t)need;
            if (overlaps(ws->ptr, wb, d->q, q_bytes) || overlaps(ws->ptr, wb, d->k, k_bytes) ||
                overlaps(ws->ptr, wb, d->v, v_bytes) || overlaps(ws->ptr, wb, d->cos, tab_bytes) ||
                overlaps(ws->ptr, wb, d->sin, tab_bytes) || overlaps(ws->ptr, wb, d->out, out_bytes))
                return SA3_ERR_ARG;
        }
        a.ws = ws->ptr;
        a.prep = 1;
        a.run_prep = ws->policy != SA3_PREP_REUSE;
        a.run_main = ws->policy != SA3_PREP_ONLY;
        if ((((unsigned long long)d->L + 63) / 64) * bh >= (1ull << 31)) return SA3_ERR_SHAPE;
    }

    const unsigned long long tiles = ((unsigned long long)d->L + sa3::tile_rows(a) - 1) / sa3::tile_rows(a);
    if (tiles * bh >= (1ull << 31)) return SA3_ERR_SHAPE;

    const int dev = check_device();
    if (dev != SA3_OK) return dev;
    // the static scratch: this device's address of the array (never its host-side name)
    if (a.prep && ws->scratch && sa3::scratch_device_ptr(&a.ws) != 0) return SA3_ERR_DEVICE;

    const int e = sa3::launch_forward(a);
    return e == (int)hipSuccess ? SA3_OK : SA3_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int sa3attn_forward_ex(const sa3attn_desc *desc) { return forward_impl(desc, nullptr, nullptr); }

int sa3attn_forward_strided(const sa3attn_desc *desc, const sa3attn_strides *strides) {
    if (!strides) return SA3_ERR_NULL;
    return forward_impl(desc, strides, nullptr);
}

int sa3attn_forward_general(const sa3attn_desc *desc, const sa3attn_strides *strides, const sa3attn_rope *rope) {
    return forward_impl(desc, strides, rope);
}

int sa3attn_workspace_bytes(const sa3attn_desc *desc, int policy, unsigned long long *bytes) {
    if (!desc || !bytes) return SA3_ERR_NULL;
    const int shape = check_shape(desc);
    if (shape != SA3_OK) return shape;
    if (!policy_ok(policy)) return SA3_ERR_ARG;
    sa3::LaunchArgs a{};
    shape_args(desc, a);
    *bytes = prep_need(a, policy);
    return SA3_OK;
}

int sa3attn_forward_ws(const sa3attn_desc *desc, const sa3attn_strides *strides, const sa3attn_rope *rope,
                       void *workspace, unsigned long long workspace_bytes, int policy) {
    const Workspace w{workspace, workspace_bytes, policy, false};
    return forward_impl(desc, strides, rope, &w);
}

int sa3attn_forward_noalloc(const sa3attn_desc *desc, const sa3attn_strides *strides, const sa3attn_rope *rope,
                            int policy) {
    const Workspace w{nullptr, sa3::kScratchBytes, policy, true};
    return forward_impl(desc, strides, rope, &w);
}

static int forward_short(const void *q, const void *k, const void *v, const float *cos, const float *sin,
                         void *out, int B, int H, int L, int D, int window, float lambda, float scale,
                         void *stream, int dtype) {
    sa3attn_desc d;
    d.q = q;
    d.k = k;
    d.v = v;
    d.cos = cos;
    d.sin = sin;
    d.out = out;
    d.B = B;
    d.H = H;
    d.L = L;
    d.D = D;
    d.window = window;
    d.lambda = lambda;
    d.scale = scale;
    d.dtype = dtype;
    d.out_dtype = dtype;
    d.differential = lambda != 0.0f ? 1 : 0;
    d.stream = stream;
    return forward_impl(&d, nullptr, nullptr);
}

int sa3attn_forward(const void *q, const void *k, const void *v, const float *cos, const float *sin, void *out,
                    int B, int H, int L, int D, int window, float lambda, float scale, void *stream) {
    return forward_short(q, k, v, cos, sin, out, B, H, L, D, window, lambda, scale, stream, SA3_F16);
}

int sa3attn_forward_bf16(const void *q, const void *k, const void *v, const float *cos, const float *sin,
                         void *out, int B, int H, int L, int D, int window, float lambda, float scale,
                         void *stream) {
    return forward_short(q, k, v, cos, sin, out, B, H, L, D, window, lambda, scale, stream, SA3_BF16);
}

const char *sa3attn_status_string(int status) {
    switch (status) {
        case SA3_OK: return "SA3_OK";
        case SA3_ERR_NULL: return "SA3_ERR_NULL: a required pointer is NULL";
        case SA3_ERR_SHAPE: return "SA3_ERR_SHAPE: B, H, L or D out of range, D odd, or a size overflows";
        case SA3_ERR_UNSUPPORTED: return "SA3_ERR_UNSUPPORTED: head dim (64 or 128) or dtype not supported";
        case SA3_ERR_ARG:
            return "SA3_ERR_ARG: non-finite scale or lambda, out overlaps an input, a misaligned pointer, "
                   "or unusable strides";
        case SA3_ERR_DEVICE: return "SA3_ERR_DEVICE: no HIP device, or the current device is not gfx950";
        case SA3_ERR_LAUNCH: return "SA3_ERR_LAUNCH: kernel launch failed";
        case SA3_ERR_SCRATCH:
            return "SA3_ERR_SCRATCH: the pre-pass workspace of this call exceeds the static scratch of "
                   "sa3attn_forward_noalloc (SA3ATTN_SCRATCH_BYTES)";
        default: return "unknown sa3attn status";
    }
}

int sa3attn_version(void) { return (SA3ATTN_VERSION_MAJOR << 16) | SA3ATTN_VERSION_MINOR; }

}  // extern "C"
