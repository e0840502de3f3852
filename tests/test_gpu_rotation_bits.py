"""GPU: the rotated K and the fp16 V tiles, bit for bit against the oracle.

The method rotates Q and K in FP32 and casts the result back to the activation dtype
before QK^T ("Fixes the medium DiT's FP16-mixed ONNX ..." discussion, sections "The
bug" and "The fix"). The end-to-end parity tests see that cast only through the 2e-3
bar, which a contracted (fused multiply-add) rotation would still pass. The pre-pass
writes exactly the QK^T operands the attention kernel uses (K' per branch, in the IO
type) and the P.V operands (V converted to fp16, each 64-key tile transposed with bits
2 and 3 of the key index swapped) into the caller's workspace; the "only" policy runs
it alone. Here that workspace is read back and compared bit for bit with the oracle's
FP32 rotation and cast (oracle.rotate_method) and with an exact fp16 conversion of V
put in the tile layout by hand; rows past L must be zeros.
"""

import numpy as np
import pytest

import oracle
from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _bits(x64, io):
    """IO-dtype values (fp64 array holding exact IO values) -> uint16 bit patterns."""
    if io == "f16":
        return x64.astype(np.float16).view(np.uint16)
    return oracle.f32_to_bf16_bits(x64.astype(np.float32))


def _swap23(p):
    return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1)


CASES = [
    # io, pairing, rotary dim R, head dim D, L, differential
    ("f16", "adjacent", 64, 64, 8192, False),
    ("bf16", "adjacent", 64, 64, 8192, False),
    ("f16", "half", 64, 64, 3000, False),
    ("bf16", "half", 32, 64, 3001, False),
    ("f16", "adjacent", 16, 64, 1000, False),
    ("bf16", "adjacent", 64, 64, 1500, True),
    ("bf16", "adjacent", 128, 128, 4096, False),
    ("f16", "half", 128, 128, 2000, False),
    ("bf16", "half", 96, 128, 1500, False),
    ("f16", "adjacent", 32, 128, 1000, True),
]


@pytest.mark.parametrize("io,pairing,R,D,L,diff", CASES)
def test_prepass_workspace_bits(io, pairing, R, D, L, diff):
    torch = G.torch_mod()
    base = "samel_swa" if diff else "dit_2min"
    cfg = synth.config(base, B=1, H=2, L=L, D=D, io=io, out="f32", window=-1, seed=31000 + L + R)
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], io) for n in ("q", "k", "v"))
    c, s = G.device_table(L, R, cfg.base)
    nb = G.sa3.workspace_bytes(cfg.B, cfg.H, L, D, differential=diff, dtype=G.sa3.BF16 if io == "bf16" else G.sa3.F16,
                               out_dtype=G.sa3.F32, prep="always")
    assert nb > 0
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda")
    out = torch.full((cfg.B, cfg.H, L, D), 7.0, dtype=torch.float32, device="cuda")
    G.note(f"  rotation bits: {io} {pairing} R={R} D={D} L={L} diff={diff}")
    G.sa3.forward(q, k, v, c, s, lam=cfg.lam, scale=cfg.scale, out=out, differential=diff, pairing=pairing,
                  rotary_dim=R, prep="only", workspace=ws)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "the pre-pass alone wrote out"
    w = ws.cpu().numpy().view(np.uint16)

    nbr, BH, Lp = (2 if diff else 1), cfg.B * cfg.H, (L + 63) // 64 * 64
    kw = w[:nbr * BH * Lp * D].reshape(nbr, BH, Lp, D)
    vw = w[nbr * BH * Lp * D:(nbr + 1) * BH * Lp * D].reshape(BH, Lp // 64, D, 64)

    c32, s32 = oracle.rope_table_f32(L, R, cfg.base)
    kk = oracle.widen_io(inp["k"], io).reshape(nbr, BH, L, D)
    for br in range(nbr):
        want = _bits(oracle.rotate_method(kk[br], c32, s32, io, pairing=pairing, rotary_dim=R), io)
        got = kw[br, :, :L, :]
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"K' branch {br}: {len(bad)} elements differ, first at {tuple(bad[0])}: "
                               f"got {got[tuple(bad[0])]:#06x} want {want[tuple(bad[0])]:#06x}")
        assert not kw[br, :, L:, :].any(), "K' rows past L are not zero"

    # V': fp16 of v (exact for these values), tile t, row d, position p <- key 64 t + swap23(p)
    vv = oracle.widen_io(inp["v"], io).reshape(BH, L, D)
    vpad = np.zeros((BH, Lp, D), dtype=np.float64)
    vpad[:, :L] = vv
    keys = np.arange(Lp).reshape(Lp // 64, 64)
    keys = keys[:, _swap23(np.arange(64))]                                   # [tile, position]
    want_v = vpad[:, keys, :].transpose(0, 1, 3, 2).astype(np.float16).view(np.uint16)   # [BH, tile, D, 64]
    bad = np.argwhere(vw != want_v)
    assert bad.size == 0, f"V': {len(bad)} elements differ, first at {tuple(bad[0])}"
