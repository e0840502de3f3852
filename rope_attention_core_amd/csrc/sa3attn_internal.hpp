// Internal interface between the C-ABI layer (api.cpp) and the gfx950 kernels
// (attn_fwd.hip, attn_narrow.hip). Not installed; not part of the public header.
#pragma once

#include <cstdint>

namespace sa3 {

// Fully validated launch description. Pointers are device pointers.
struct LaunchArgs {
    const void *q;          // [B][H][L][64] (stacked [2][...] when diff)
    const void *k;          // same layout as q
    const void *v;          // [B][H][L][64]
    const float *cos;       // [>=L][32]
    const float *sin;       // [>=L][32]
    void *out;              // [B][H][L][64]
    int B, H, L;
    int window;             // half-width; -1 = full (normalised: window < L - 1)
    float lam;              // differential weight
    float scale_log2;       // |scale| * log2(e), >= 0
    int neg_scale;          // scale < 0: q is negated on load (exact)
    int dtype;              // SA3_F16 / SA3_BF16
    int out_dtype;          // SA3_F16 / SA3_BF16 / SA3_F32
    int diff;               // two branches
    void *stream;           // hipStream_t
};

// Picks the kernel instance and launches it. Returns a hipError_t value.
int launch_forward(const LaunchArgs &a);

// Query rows handled by one workgroup of the instance launch_forward picks, so the
// host can check the grid size before launching.
int tile_rows(const LaunchArgs &a);

// The single-span kernel (sequences of <= 256 keys, or windows of half-width <= 32):
// whether it takes this call, its launcher and its query rows per workgroup.
bool narrow_applies(const LaunchArgs &a);
int launch_narrow(const LaunchArgs &a);
int narrow_tile_rows(const LaunchArgs &a);

}  // namespace sa3
