"""GPU checks of the pre-pass path (sa3attn_forward_ws through the binding).

The pre-pass rotates K and converts / transposes V once into a workspace; the
long-span kernel then copies its key tiles from there. The arithmetic per element is
the same, so the cases here give the same bits as the fused path (prep="never"),
except plain full attention on under-filled grids (the key-split kernel), grids whose
last round is split, and plain D = 64 one-round grids (128-key steps), whose sums run
in another order: both paths are then compared with the oracle. Results are also
compared with the oracle element by element on a subset. Cases cover plain and
differential attention, full and wide windows, both IO dtypes, ragged lengths (the
workspace's tail rows), strided views, the RoPE options, head dim 128, a workspace
full of NaN bits on entry, reuse of one workspace by calls of different shapes, graph
capture, and a workspace the binding allocates for a call queued on another stream.
"""

import numpy as np
import pytest

import oracle
from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _inputs(cfg, strided=False):
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    if strided:
        q, k, v = (t.transpose(-2, -3).contiguous().transpose(-2, -3) for t in (q, k, v))
    return inp, q, k, v


def _call(cfg, q, k, v, rd=None, pairing="adjacent", **kw):
    c, s = G.device_table(cfg.L, rd or cfg.D, cfg.base)
    return G.sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale,
                         out_dtype=G.out_torch_dtype(cfg.out_dtype), differential=cfg.diff,
                         pairing=pairing, rotary_dim=rd, **kw)


CASES = [
    # name, overrides, strided, (pairing, rotary_dim) or None
    ("dit_2min", dict(H=3, L=700), False, None),                           # plain, ragged
    ("dit_2min", dict(H=2, L=1000, io="bf16", out="f32"), False, None),     # bf16 V conversion
    ("dit_2min_prime", dict(H=2), False, None),                             # L = 1291
    ("samel_swa", dict(H=2, L=900, window=-1), False, None),                # differential
    ("samel_swa", dict(H=2, L=1500, window=200), False, None),              # differential, windowed
    ("dit_2min", dict(H=2, L=800, window=100, io="bf16", out="bf16"), False, None),
    ("dit_2min", dict(H=3, L=700), True, None),                             # [B, L, H, D] views
    ("samel_swa", dict(H=2, L=700, window=-1), True, ("half", 32)),         # views + RoPE options
    ("dit_2min", dict(H=2, L=600), False, ("half", 64)),
    ("dit_2min", dict(H=2, L=600), False, ("adjacent", 48)),
    ("dit_2min", dict(H=2, L=700, D=128), False, None),                     # head dim 128
    ("samel_swa", dict(H=2, L=600, window=-1, D=128), False, None),
    ("dit_2min", dict(H=2, L=500, D=128), True, ("half", 96)),
    ("dit_2min", dict(H=2, L=300), False, None),                            # two key tiles past 256
]


def _rope_kw(opt):
    return {} if opt is None else dict(pairing=opt[0], rd=opt[1])


def _takes_split_kernel(cfg, strided, opt):
    """Plain full attention at D = 64 on contiguous tensors whose grid of 256-row tiles
    leaves CUs idle and whose 64-row tiles fit one round (two per CU on 256 CUs): with
    the pre-pass these run the key-split kernel, whose sums over a row's keys are taken
    in two halves and so differ from the fused path's in the last bits."""
    bh = cfg.B * cfg.H
    full = cfg.window < 0 or cfg.window >= cfg.L - 1
    return (not strided and opt is None and cfg.D == 64 and not cfg.diff and full and cfg.L > 256
            and (cfg.L + 255) // 256 * bh < 256 and (cfg.L + 63) // 64 * bh <= 512)


def _oracle_opt(cfg, inp, opt):
    """The oracle with a RoPE option (pairing, rotary width)."""
    pairing, rd = opt
    q, k, v = G.widen(inp, cfg)
    c32, s32 = oracle.rope_table_f32(cfg.L, rd, cfg.base)
    kw = dict(pairing=pairing, rotary_dim=rd)
    if cfg.diff:
        return oracle.attn_method(q[0], k[0], v, c32, s32, cfg.io, cfg.scale, window=cfg.window, lam=cfg.lam,
                                  q2=q[1], k2=k[1], **kw)
    return oracle.attn_method(q, k, v, c32, s32, cfg.io, cfg.scale, window=cfg.window, **kw)


def _takes_tail(cfg):
    """Whether the call's grid splits its last round (the split tail), which the library
    reports as workspace beyond K' and V': its ranges are merged in another order than
    the fused path's single pass, so the last bits differ (both held to the oracle)."""
    kv = (3 if cfg.diff else 2) * cfg.B * cfg.H * ((cfg.L + 63) // 64 * 64) * cfg.D * 2
    return G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, window=cfg.window, differential=cfg.diff,
                                 prep="always") > kv


@pytest.mark.parametrize("name,kw,strided,opt", CASES)
def test_prep_path_equals_fused_path(name, kw, strided, opt):
    torch = G.torch_mod()
    cfg = synth.config(name, seed=9800 + kw.get("L", 0), **kw)
    inp, q, k, v = _inputs(cfg, strided)
    G.note(f"  prep: {name} {kw} strided={strided} rope={opt}")
    fused = _call(cfg, q, k, v, prep="never", **_rope_kw(opt))
    pre = _call(cfg, q, k, v, prep="always", **_rope_kw(opt))
    torch.cuda.synchronize()
    if _takes_split_kernel(cfg, strided, opt) or _takes_tail(cfg):
        # same arithmetic per element, row sums in another order: both against the oracle
        want = G.run_oracle(cfg, inp) if opt is None else _oracle_opt(cfg, inp, opt)
        for what, got in (("key-split or split tail", pre), ("fused", fused)):
            G.assert_parity(got.float().cpu().numpy().astype(np.float64), want, what=f"{name} {kw} {what}",
                            out=cfg.out_dtype)
        return
    assert torch.equal(pre, fused), f"{name} {kw}: pre-pass path differs from the fused path"


@pytest.mark.parametrize("name,kw", [("dit_2min", dict(H=3, L=700)), ("samel_swa", dict(H=2, L=900, window=-1)),
                                     ("dit_2min", dict(H=2, L=700, D=128))])
def test_prep_path_parity(name, kw):
    cfg = synth.config(name, seed=9850, **kw)
    inp, q, k, v = _inputs(cfg)
    got = _call(cfg, q, k, v, prep="always")
    G.torch_mod().cuda.synchronize()
    G.assert_parity(got.float().cpu().numpy().astype(np.float64), G.run_oracle(cfg, inp),
                    what=f"prep {name} {kw}", out=cfg.out_dtype)


@pytest.mark.parametrize("name", ["dit_long", "dit_medium_diff", "dit_long_d128"])
def test_auto_policy_at_full_size(name):
    """The benchmark shapes: AUTO runs the pre-pass there, and matches the fused path."""
    torch = G.torch_mod()
    cfg = synth.config(name)
    assert G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, window=cfg.window, differential=cfg.diff) > 0
    inp, q, k, v = _inputs(cfg)
    fused = _call(cfg, q, k, v, prep="never")
    auto = _call(cfg, q, k, v, prep="auto")
    torch.cuda.synchronize()
    # plain D = 64 one-round grids walk the keys 128 at a time with the pre-pass, and the
    # long latent at D = 128 splits its last round: both sum in another order
    if cfg.diff:
        assert torch.equal(auto, fused)
    else:
        d = (auto.float() - fused.float()).abs().max().item()
        G.note(f"  {name}: auto vs fused max-abs difference {d:.3e}")
        assert d <= 2 * G.ATOL
    rows = np.array([0, 1, 777, cfg.L - 1])
    want = G.run_oracle_rows(cfg, inp, cfg.B - 1, cfg.H - 1, rows)
    G.assert_parity(auto[cfg.B - 1, cfg.H - 1, rows].float().cpu().numpy().astype(np.float64), want,
                    what=f"{name} auto", out=cfg.out_dtype)


def test_workspace_contents_on_entry_do_not_matter():
    """A workspace full of NaN bits, reused by a larger then a smaller call."""
    torch = G.torch_mod()
    big = synth.config("samel_swa", H=2, L=1000, window=-1, seed=9870)
    small = synth.config("dit_2min", H=1, L=333, seed=9871)
    nb = G.sa3.workspace_bytes(big.B, big.H, big.L, big.D, differential=True, dtype=G.sa3.BF16, prep="always")
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    for cfg in (big, small):
        _, q, k, v = _inputs(cfg)
        # the same call on a zeroed workspace of its own (the small plain grid takes the
        # key-split kernel with the pre-pass, so the fused path's bits are not the bar)
        clean = _call(cfg, q, k, v, prep="always",
                      workspace=torch.zeros((nb,), dtype=torch.uint8, device="cuda"))
        pre = _call(cfg, q, k, v, prep="always", workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(pre, clean), cfg.name


def test_too_small_workspace_is_rejected_and_out_untouched():
    torch = G.torch_mod()
    cfg = synth.config("dit_2min", H=2, L=700, seed=9872)
    _, q, k, v = _inputs(cfg)
    nb = G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, prep="always")
    ws = torch.empty((nb - 16,), dtype=torch.uint8, device="cuda")
    out = torch.full_like(v, 7.0)
    with pytest.raises(G.sa3.SA3Error):
        _call(cfg, q, k, v, prep="always", workspace=ws, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_prep_path_in_a_graph():
    """Two kernels captured into one graph; every replay matches the eager result."""
    torch = G.torch_mod()
    cfg = synth.config("samel_swa", H=2, L=1000, window=-1, seed=9873)
    _, q, k, v = _inputs(cfg)
    eager = _call(cfg, q, k, v, prep="always")
    nb = G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, differential=True, dtype=G.sa3.BF16, prep="always")
    ws = torch.empty((nb,), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(eager)
    c, s = G.device_table(cfg.L, cfg.D, cfg.base)
    call = dict(window=cfg.window, lam=cfg.lam, scale=cfg.scale, out=out, differential=True, prep="always",
                workspace=ws)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(2):
            G.sa3.forward(q, k, v, c, s, **call)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.sa3.forward(q, k, v, c, s, **call)
    for i in range(4):
        out.zero_()
        ws.fill_(0xFF if i % 2 else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from eager"


def test_prepare_once_then_reuse_for_several_queries():
    """The "only" policy fills the workspace from k, v; "reuse" runs the attention
    kernel alone on it, for the original q and for a second q against the same keys."""
    torch = G.torch_mod()
    cfg = synth.config("samel_swa", H=2, L=800, window=-1, seed=9874)
    _, q, k, v = _inputs(cfg)
    q2 = torch.flip(q, dims=[-2]).contiguous()
    nb = G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, differential=True, prep="always")
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.full((cfg.B, cfg.H, cfg.L, cfg.D), 7.0, dtype=torch.float32, device="cuda")
    _call(cfg, q, k, v, prep="only", workspace=ws, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "the pre-pass alone wrote out"
    for qq in (q, q2):
        want = _call(cfg, qq, k, v, prep="always")
        got = _call(cfg, qq, k, v, prep="reuse", workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, want)


def test_internal_workspace_on_a_side_stream():
    """The binding allocates the workspace (on torch's current stream) for a call queued
    on another stream: it stays reserved until that stream has run the call, so
    same-sized blocks allocated and filled on the current stream meanwhile leave the
    results equal to those of the same call on the current stream."""
    torch = G.torch_mod()
    cfg = synth.config("dit_2min", H=4, L=2000, seed=9880)
    _, q, k, v = _inputs(cfg)
    fused = _call(cfg, q, k, v, prep="always")
    torch.cuda.synchronize()
    nb = G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, prep="always")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs, fills = [], []
    for i in range(3):
        out = torch.empty_like(fused)
        _call(cfg, q, k, v, prep="always", out=out, stream=side)
        fills.append(torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda"))
        outs.append(out)
    torch.cuda.synchronize()
    for i, out in enumerate(outs):
        assert torch.equal(out, fused), f"call {i} on the side stream differs"


@pytest.mark.parametrize("prep", ["only", "reuse"])
def test_only_and_reuse_need_a_workspace(prep):
    """Without the caller's workspace, "reuse" would read an uninitialised one and
    "only" would fill one that is dropped: both raise, and out is untouched."""
    torch = G.torch_mod()
    cfg = synth.config("dit_2min", H=2, L=700, seed=9890)
    _, q, k, v = _inputs(cfg)
    out = torch.full_like(v, 7.0)
    with pytest.raises(ValueError):
        _call(cfg, q, k, v, prep=prep, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
