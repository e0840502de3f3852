// Internal interface between the C-ABI layer (api.cpp) and the gfx950 kernels
// (attn_fwd.hip, attn_narrow.hip). Not installed; not part of the public header.
#pragma once

#include <cstdint>

#include "sa3attn.h"

namespace sa3 {

// Fully validated launch description. Pointers are device pointers.
struct LaunchArgs {
    const void *q;          // element (b, h, l, d) at b*qs[0] + h*qs[1] + l*qs[2] + d (+ q_br: branch 2)
    const void *k;          // likewise with ks and k_br
    const void *v;          // likewise with vs
    const float *cos;       // [>=L][R/2]
    const float *sin;       // [>=L][R/2]
    void *out;              // likewise with os
    long long qs[3], ks[3], vs[3], os[3];   // element strides of b, h, l (d is contiguous)
    long long q_br, k_br;   // elements from branch 1 to branch 2 (differential)
    int B, H, L;
    int D;                  // head dim: 64 or 128
    int window;             // half-width; -1 = full (normalised: window < L - 1)
    float lam;              // differential weight
    float scale_log2;       // |scale| * log2(e), >= 0
    int neg_scale;          // scale < 0: q is negated on load (exact)
    int dtype;              // SA3_F16 / SA3_BF16
    int out_dtype;          // SA3_F16 / SA3_BF16 / SA3_F32
    int diff;               // two branches
    int contig;             // contiguous [B][H][L][D] (and stacked [2][...]), adjacent pairs, R = D
    int rope_half;          // RoPE pairs (x[i], x[i + R/2]) instead of (x[2i], x[2i+1])
    int rot_dim;            // R: leading dims rotated (multiple of 16, <= D); the table has R/2 columns
    void *ws;               // workspace of the pre-pass (prep_bytes(a) bytes), or nullptr
    int prep;               // the long-span kernel reads K and V from the pre-pass workspace
    int run_prep;           // with prep: enqueue the pre-pass (0: ws already holds its result)
    int run_main;           // enqueue the attention kernel (0: only the pre-pass)
    int n_cu;               // compute units of the current device (256 when there is none)
    int tail_ok;            // with prep: the workspace may also hold the split tail's partials
    void *stream;           // hipStream_t
};

// Picks the kernel instance and launches it. Returns a hipError_t value.
int launch_forward(const LaunchArgs &a);

// Query rows handled by one workgroup of the instance launch_forward picks, so the
// host can check the grid size before launching.
int tile_rows(const LaunchArgs &a);

// The key-split kernel (attn_split.hip) for such grids under plain full attention with
// the pre-pass (contiguous, default RoPE): whether it applies, and its launcher.
bool split_applies(const LaunchArgs &a);
int launch_split(const LaunchArgs &a, int n_qtiles);

// Whether the single-span kernel takes the call (D = 64 only).
bool use_narrow(const LaunchArgs &a);

// Plain D = 64 calls whose grid of 256-row tiles has fewer workgroups than
// compute units: with the pre-pass they run 64-row tiles of 2-wave workgroups.
bool small_grid(const LaunchArgs &a);

// The pre-pass (attn_prep.hip): K of each branch rotated and V converted to fp16 and
// transposed, once per key tile, into a workspace the long-span kernel then copies
// from. prep_bytes: the workspace it needs (0 when the call takes the single-span
// kernel, which has no use for it); prep_pays: whether the saving in the long-span
// kernel (each key tile is rotated by every query tile that visits it) outweighs the
// extra pass; launch_prep: enqueues it (a.ws set).
unsigned long long prep_bytes(const LaunchArgs &a);

// The split tail of the long-span kernel: a grid of one workgroup per query tile whose
// last round would leave at least half the compute units idle splits each of its last
// n_tail tiles into k key ranges (n_full whole tiles before them). k = 0: no split.
// Applies with the pre-pass when a.tail_ok: its workspace holds, after K' and V', the
// partial results (from byte part_off) and one counter per split tile (from cnt_off),
// which the pre-pass clears.
struct TailPlan {
    int n_full, k, n_tail;
    unsigned long long part_off, cnt_off, end;   // byte offsets in the workspace; end: its size
};
TailPlan tail_plan(const LaunchArgs &a);
bool prep_pays(const LaunchArgs &a);
int launch_prep(const LaunchArgs &a);

// The single-span kernel (sequences of <= 256 keys, or windows of half-width <= 32):
// whether it takes this call, its launcher and its query rows per workgroup.
bool narrow_applies(const LaunchArgs &a);
int launch_narrow(const LaunchArgs &a);
int narrow_tile_rows(const LaunchArgs &a);

// The static device scratch (scratch.hip) that sa3attn_forward_noalloc uses as the
// pre-pass workspace: its size, and the current device's address of it (looked up once
// per device with hipGetSymbolAddress; returns 0, or -1 when there is no usable device).
constexpr unsigned long long kScratchBytes = SA3ATTN_SCRATCH_BYTES;
int scratch_device_ptr(void **ptr);

}  // namespace sa3
