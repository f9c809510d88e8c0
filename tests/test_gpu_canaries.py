"""Every output buffer is followed by guard bytes of a known pattern; after each
entry point runs (on ragged shapes that exercise the kernels' tail handling),
the guard bytes must be unchanged: no kernel writes past the end of an output.
The results themselves are checked against the oracle in the other GPU tests."""
import numpy as np
import pytest

import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu

GUARD = 4096   # bytes
PATTERN = 0xA5


class Guarded:
    """A contiguous tensor of `shape` and `dtype` followed by GUARD pattern bytes."""

    def __init__(self, shape, dtype):
        import torch
        item = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * item
        self.n = n
        self.raw = torch.full((n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[:n].view(dtype).view(shape)

    def intact(self):
        import torch
        torch.cuda.synchronize()
        tail = self.raw[self.n:].cpu().numpy()
        return bool(np.all(tail == PATTERN))


def _plane_shape(fmt, N, K):
    import torch
    return {"int4": ((N, K // 32), torch.uint16), "fp4": ((N, K // 32), torch.uint8),
            "int8": ((N, K // 32), torch.uint16), "km4": ((N, 16), torch.uint16),
            "int4aff": ((N, K // 32), torch.int32), "int8km": ((N // 32, 256), torch.uint16)}[fmt]


def _codes_shape(fmt, N, K):
    import torch
    return (N, K if fmt in ("int8", "int8km") else K // 2), (torch.int8 if fmt == "int8" else torch.uint8)


@pytest.mark.parametrize("fmt", ["int4", "fp4", "int8", "km4", "int4aff", "int8km"])
def test_pack_matvec_dequant_write_nothing_past_their_outputs(fmt):
    import torch
    for N, K in ((1037, 1056), (8192 + 13, 2048), (32768 + 37, 1024)):
        if fmt == "int8km":
            N -= N % 32
        c = wl.small_dense(fmt, N, K, batch=8, seed=N, outlier_frac=0.01)
        W = dev(c.W)
        cs, cd = _codes_shape(fmt, N, K)
        ps, pd = _plane_shape(fmt, N, K)
        gc, gp = Guarded(cs, cd), Guarded(ps, pd)
        if fmt == "int4":
            qmv.qpack_int4(W, codes=gc.t, scale=gp.t)
        elif fmt == "fp4":
            qmv.qpack_fp4(W, codes=gc.t, scale=gp.t)
        elif fmt == "int8":
            qmv.qpack_int8(W, codes=gc.t, scale=gp.t)
        elif fmt == "km4":
            qmv.qpack_km4(W, codes=gc.t, lut=gp.t)
        elif fmt == "int4aff":
            qmv.qpack_int4aff(W, codes=gc.t, plane=gp.t)
        else:
            qmv.qpack_int8km(W, codes=gc.t, lut=gp.t)
        assert gc.intact() and gp.intact(), (fmt, N, K, "pack")
        x = dev(c.x)
        for B in (1, 2, 3, 5, 8):
            gy = Guarded((B, N), torch.float32)
            qmv.qmatvec(fmt, gc.t, gp.t, x[:B], y=gy.t)
            assert gy.intact(), (fmt, N, K, B, "matvec")
        gd = Guarded((N, K), torch.float32)
        qmv.qdequant(fmt, gc.t, gp.t, out=gd.t)
        assert gd.intact(), (fmt, N, K, "dequant")
        for B in (1, 8):
            gi, gv = Guarded((B,), torch.int32), Guarded((B,), torch.float32)
            gw = Guarded((qmv.qmatvec_argmax_workspace_bytes(N, B),), torch.uint8)
            qmv.qmatvec_argmax(fmt, gc.t, gp.t, x[:B], idx=gi.t, val=gv.t, workspace=gw.t)
            assert gi.intact() and gv.intact() and gw.intact(), (fmt, N, K, B, "argmax")
            qmv.qmatvec_argmax_noalloc(fmt, gc.t, gp.t, x[:B], idx=gi.t, val=gv.t)
            assert gi.intact() and gv.intact(), (fmt, N, K, B, "argmax_noalloc")


def test_km4o_moe_embedding_and_stream_write_nothing_past_their_outputs():
    import torch
    N, K, P = 1037, 1056, 5
    c = wl.small_dense("km4", N, K, batch=8, seed=3)
    packed = qmv.qpack_km4o(dev(c.W), P)
    for B in (1, 4, 8):
        gy = Guarded((B, N), torch.float32)
        qmv.qmatvec_km4o(*packed, dev(c.x[:B]), y=gy.t)
        assert gy.intact(), ("km4o", B)
    # MoE: 16 experts, H = 256, I = 96 (ragged against the kernels' row groups)
    E, H, I, T, topk = 16, 256, 96, 5, 4
    rng = np.random.default_rng(9)
    gu = (rng.standard_normal((E * 2 * I, H)) * 0.02).astype(np.float16)
    dn = (rng.standard_normal((E * H, I)) * 0.02).astype(np.float16)
    for fmt in ("int4", "fp4", "int4aff"):
        guc, gup = qmv.qpack(fmt, dev(gu))
        dnc, dnp = qmv.qpack(fmt, dev(dn))
        guc, gup = guc.view(E, 2 * I, -1), gup.view(E, -1)
        dnc, dnp = dnc.view(E, H, -1), dnp.view(E, -1)
        x = dev(rng.standard_normal((T, H)).astype(np.float16))
        lg = dev(rng.standard_normal((T, E)).astype(np.float32))
        gi, gw = Guarded((T, topk), torch.int32), Guarded((T, topk), torch.float32)
        qmv.qmoe_route(lg, topk, ids=gi.t, weights=gw.t)
        assert gi.intact() and gw.intact(), (fmt, "route")
        gh = Guarded((T, topk, I), torch.float16)
        qmv.gather_qmatvec(fmt, guc, gup, x, gi.t, epi="swiglu", y=gh.t)
        assert gh.intact(), (fmt, "swiglu")
        gn = Guarded((T, topk, 2 * I), torch.float32)
        qmv.gather_qmatvec(fmt, guc, gup, x, gi.t, epi="none", y=gn.t)
        assert gn.intact(), (fmt, "none")
        gc_ = Guarded((T, H), torch.float32)
        qmv.gather_qmatvec(fmt, dnc, dnp, gh.t, gi.t, weights=gw.t, epi="combine", x_per_slot=True, y=gc_.t)
        assert gc_.intact(), (fmt, "combine")
        for tt in (1, T):
            g = [Guarded((tt, topk), torch.int32), Guarded((tt, topk), torch.float32),
                 Guarded((tt, topk, I), torch.float16), Guarded((tt, H), torch.float32)]
            qmv.qmoe_ffn(fmt, guc, gup, dnc, dnp, x[:tt].contiguous(), lg[:tt].contiguous(), topk,
                         ids=g[0].t, weights=g[1].t, h=g[2].t, y=g[3].t)
            assert all(v.intact() for v in g), (fmt, tt, "ffn")
    # int8 embedding table
    q, s = qmv.qpack_int8_rows(dev(c.W))
    go = Guarded((7, K), torch.float16)
    qmv.qembed_gather_int8(q, s, dev(np.array([0, 5, -1, N, N - 1, 3, 3], np.int32)), out=go.t)
    assert go.intact()
    # streaming read: the sink holds exactly one word per workgroup
    buf = torch.randint(0, 255, (1 << 20,), dtype=torch.uint8, device="cuda")
    words = int(qmv.lib().qmv_stream_read_sink_words(buf.numel()))
    gs = Guarded((words,), torch.int32)
    qmv.qmv_stream_read(buf, sink=gs.t)
    assert gs.intact()


def test_tiled_km4_writes_nothing_past_its_outputs():
    import torch
    rng = np.random.default_rng(11)
    for N, K in ((37, 512), (1037, 2048), (66000 + 5, 1024)):
        codes = dev(rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8))
        lut = dev((rng.standard_normal((N, 16)) * 0.02).astype(np.float16).view(np.uint16))
        gt = Guarded((qmv.qtile_km4_bytes(N, K),), torch.uint8)
        qmv.qtile_km4(codes, tiled=gt.t)
        assert gt.intact(), ("tile", N, K)
        for B in (1, 2, 4):
            xb = dev(rng.standard_normal((B, K)).astype(np.float16))
            gy = Guarded((B, N), torch.float32)
            qmv.qmatvec_km4_tiled(gt.t, lut, xb, y=gy.t)
            assert gy.intact(), ("tiled matvec", N, K, B)
            gi, gv = Guarded((B,), torch.int32), Guarded((B,), torch.float32)
            gw = Guarded((qmv.qmatvec_argmax_workspace_bytes(N, B),), torch.uint8)
            qmv.qmatvec_argmax_km4_tiled(gt.t, lut, xb, idx=gi.t, val=gv.t, workspace=gw.t)
            assert gi.intact() and gv.intact() and gw.intact(), ("tiled argmax", N, K, B)
