"""GPU: sa3attn_forward_noalloc against sa3attn_forward_ws, through the C-ABI.

sa3attn_forward_noalloc is for callers that cannot allocate device memory: the
pre-pass workspace is the library's static device array instead of a caller buffer.
Its outputs must be bitwise those of sa3attn_forward_ws with a workspace of the
caller's (same kernels, same arithmetic), call after call: here a full-size call
(the long latent, 48 MiB of workspace) and then a smaller one, whose pre-pass
overwrites only the start of the array, plus the "only" / "reuse" pair and the size
limit. Torch's allocator must see no allocation during the no-alloc calls.
"""

import ctypes

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu

AUTO, ALWAYS, NEVER, ONLY, REUSE = 0, 1, 2, 3, 4
SA3_ERR_SCRATCH = -7


def _setup(cfg):
    torch = G.torch_mod()
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    c, s = G.device_table(cfg.L, cfg.D, cfg.base)
    odt = G.out_torch_dtype(cfg.out_dtype)
    outs = [torch.full((cfg.B, cfg.H, cfg.L, cfg.D), float("nan"), dtype=odt, device="cuda") for _ in range(2)]
    return inp, (q, k, v, c, s), outs


def _desc(cfg, t, out):
    q, k, v, c, s = t
    io = G.sa3.BF16 if cfg.io == "bf16" else G.sa3.F16
    od = {"f16": G.sa3.F16, "bf16": G.sa3.BF16, "f32": G.sa3.F32}[cfg.out_dtype]
    stream = G.torch_mod().cuda.current_stream().cuda_stream
    return G.sa3._Desc(q.data_ptr(), k.data_ptr(), v.data_ptr(), c.data_ptr(), s.data_ptr(), out.data_ptr(),
                       cfg.B, cfg.H, cfg.L, cfg.D, cfg.window, cfg.lam, cfg.scale, io, od, 1 if cfg.diff else 0,
                       stream)


def _ws_call(lib, cfg, t, out, policy, ws):
    d = _desc(cfg, t, out)
    return lib.sa3attn_forward_ws(ctypes.byref(d), None, None, ws.data_ptr(), ws.numel(), policy)


def _na_call(lib, cfg, t, out, policy):
    d = _desc(cfg, t, out)
    return lib.sa3attn_forward_noalloc(ctypes.byref(d), None, None, policy)


def _allocations():
    return G.torch_mod().cuda.memory_stats().get("allocation.all.allocated", 0)


def test_noalloc_matches_ws_call_after_call():
    torch = G.torch_mod()
    lib = G.sa3.load_library()
    big = synth.config("dit_long")                                   # 48 MiB of workspace
    small = synth.config("dit_2min", H=3, L=1000, io="bf16", out="f32", seed=77)
    for cfg, policies in ((big, (AUTO, ALWAYS)), (small, (ALWAYS,)), (big, (ALWAYS,))):
        inp, t, (o_ws, o_na) = _setup(cfg)
        nb = G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, window=cfg.window, differential=cfg.diff,
                                   dtype=G.sa3.BF16 if cfg.io == "bf16" else G.sa3.F16, prep="always")
        assert 0 < nb <= G.sa3.SCRATCH_BYTES
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        for policy in policies:
            G.note(f"  noalloc: {cfg.name} B{cfg.B} H{cfg.H} L{cfg.L} policy {policy}")
            o_ws.fill_(float("nan"))
            o_na.fill_(float("nan"))
            assert _ws_call(lib, cfg, t, o_ws, policy, ws) == 0
            torch.cuda.synchronize()
            before = _allocations()
            assert _na_call(lib, cfg, t, o_na, policy) == 0
            torch.cuda.synchronize()
            assert _allocations() == before, "an allocation during the no-alloc call"
            assert torch.equal(o_na, o_ws), f"{cfg.name} policy {policy}: differs from the workspace call"
        # and against the oracle on a few rows
        rows = np.array([0, 1, cfg.L // 2, cfg.L - 1])
        want = G.run_oracle_rows(cfg, inp, cfg.B - 1, cfg.H - 1, rows)
        G.assert_parity(o_na[cfg.B - 1, cfg.H - 1, rows].float().cpu().numpy().astype(np.float64), want,
                        what=f"noalloc {cfg.name}", out=cfg.out_dtype)


def test_noalloc_only_then_reuse():
    """ONLY fills the static array from k, v; REUSE then runs the attention kernel on it."""
    torch = G.torch_mod()
    lib = G.sa3.load_library()
    cfg = synth.config("samel_swa", H=2, L=1200, window=-1, seed=78)
    _, t, (o_ref, o_na) = _setup(cfg)
    assert _na_call(lib, cfg, t, o_ref, ALWAYS) == 0
    o_na.fill_(7.0)
    assert _na_call(lib, cfg, t, o_na, ONLY) == 0
    torch.cuda.synchronize()
    assert bool((o_na == 7.0).all()), "ONLY wrote out"
    assert _na_call(lib, cfg, t, o_na, REUSE) == 0
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref)


def test_noalloc_split_tail():
    """A grid whose last round is split: with room in the static array for the partials
    (B1 H24 L3000: 27 MiB) the no-alloc call splits it as the workspace call does (the
    same bits); the long latent at D = 128 (82 MiB with the partials, 48 MiB without)
    runs the pre-pass without the split: against the oracle on the heads whose tiles
    the workspace call splits, and not the split call's bits."""
    torch = G.torch_mod()
    lib = G.sa3.load_library()
    cfg = synth.config("dit_long", B=1, H=24, L=3000, seed=80)
    inp, t, (o_ws, o_na) = _setup(cfg)
    nb = G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, dtype=G.sa3.BF16, prep="always")
    assert nb <= G.sa3.SCRATCH_BYTES
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    assert _ws_call(lib, cfg, t, o_ws, ALWAYS, ws) == 0
    assert _na_call(lib, cfg, t, o_na, ALWAYS) == 0
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws)
    big = synth.config("dit_long_d128")
    nb = G.sa3.workspace_bytes(big.B, big.H, big.L, big.D, dtype=G.sa3.BF16, prep="always")
    assert nb > G.sa3.SCRATCH_BYTES
    inp, t, (o_a, o_b) = _setup(big)
    assert _na_call(lib, big, t, o_a, ALWAYS) == 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    assert _ws_call(lib, big, t, o_b, ALWAYS, ws) == 0
    torch.cuda.synchronize()
    assert not torch.equal(o_a, o_b), "the no-alloc call split its last round"
    rows = np.array([0, 255, 256, 2049, big.L - 1])
    for b, h in ((1, 4), (1, 11)):                     # heads of the split tiles
        want = G.run_oracle_rows(big, inp, b, h, rows)
        G.assert_parity(o_a[b, h, rows].float().cpu().numpy().astype(np.float64), want,
                        what=f"noalloc d128 (b,h)=({b},{h})", out=big.out_dtype)


def test_noalloc_size_limit():
    """The medium DiT's differential shape needs 72 MiB of workspace: ALWAYS is refused
    before anything runs; AUTO runs without the pre-pass, bitwise as NEVER."""
    torch = G.torch_mod()
    lib = G.sa3.load_library()
    cfg = synth.config("dit_medium_diff")
    _, t, (o_a, o_b) = _setup(cfg)
    o_a.fill_(7.0)
    assert _na_call(lib, cfg, t, o_a, ALWAYS) == SA3_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((o_a == 7.0).all())
    assert _na_call(lib, cfg, t, o_a, AUTO) == 0
    assert _na_call(lib, cfg, t, o_b, NEVER) == 0
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)


def test_noalloc_through_the_binding():
    torch = G.torch_mod()
    cfg = synth.config("dit_2min", H=2, L=900, seed=79)
    _, (q, k, v, c, s), (o_a, o_b) = _setup(cfg)
    G.sa3.forward(q, k, v, c, s, out=o_a, prep="always")
    before = _allocations()
    G.sa3.forward_noalloc(q, k, v, c, s, o_b, prep="always")
    torch.cuda.synchronize()
    assert _allocations() == before
    assert torch.equal(o_a, o_b)
