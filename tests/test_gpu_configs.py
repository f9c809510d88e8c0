"""GPU parity at the five full workload sizes, in the launch configuration the
benchmark times (the same entry points on the same shapes):

  tiny int4   256 x 512 fp32, x fp32 [1, 512]
  fp4         4096 x 4096 fp16, x fp16 batch 1 and 4
  km4 lm_head 248320 x 2048 fp16, x fp16 batch 1 and 8
  int8 head   130560 x 2560 fp16 with heavy-tailed rows, x fp16 batch 1
  MoE         256 experts (gate/up 2 x 512 x 2048, down 2048 x 512, int4),
              top-8 routing, 1..8 tokens

The 256-expert slabs are checked on the routed experts one by one; everything
else, the k-means packing of all 248320 lm_head rows included, is compared in
full."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import RTOL, dev, host, rel_err

pytestmark = pytest.mark.gpu


def test_tiny_int4_full():
    c = wl.tiny_int4()
    codes, scale = oracle.pack_int4(c.W)
    gc, gs = qmv.qpack_int4(dev(c.W))
    assert np.array_equal(codes, host(gc)) and np.array_equal(scale, host(gs))
    y = host(qmv.qmatvec_int4(gc, gs, dev(c.x)))
    assert rel_err(y, oracle.matvec("int4", codes, scale, c.x)) <= RTOL


def test_fp4_4096_full():
    c = wl.fp4_square()
    codes, scale = oracle.pack_fp4(c.W)
    gc, gs = qmv.qpack_fp4(dev(c.W))
    assert np.array_equal(codes, host(gc)) and np.array_equal(scale, host(gs))
    for B in (1, 4):
        y = host(qmv.qmatvec_fp4(gc, gs, dev(c.x[:B])))
        assert rel_err(y, oracle.matvec("fp4", codes, scale, c.x[:B])) <= RTOL


@pytest.fixture(scope="module")
def lm_head():
    c = wl.lm_head_km4()
    W = dev(c.W)
    codes, lut = qmv.qpack_km4(W)
    del W
    # the oracle packs every row (OpenMP over rows on the host's cores)
    oc, ol = oracle.pack_km4(c.W)
    return c, codes, lut, oc, ol


def test_km4_lm_head_pack_all_rows(lm_head):
    c, codes, lut, oc, ol = lm_head
    gc, gl = host(codes), host(lut)
    bad = np.nonzero(np.any(gc != oc, axis=1) | np.any(gl != ol, axis=1))[0]
    assert bad.size == 0, "rows differing from the oracle: %s" % bad[:16]


@pytest.mark.parametrize("B", [1, 4, 8])
def test_km4_lm_head_matvec_all_rows(lm_head, B):
    """Batch 1 and 8 are the benchmarked calls; batch 4 and 8 run the
    4x4x4-block kernel (four row quads per wave at batch 4, two row quads and
    two token quads at batch 8)."""
    c, codes, lut, oc, ol = lm_head
    x = c.x[:B]
    y = host(qmv.qmatvec_km4(codes, lut, dev(x)))
    want = oracle.matvec("km4", oc, ol, x)
    assert rel_err(y, want) <= RTOL


def test_km4_lm_head_tiled_all_rows(lm_head):
    """The benchmarked call: batch 1 from the row-tiled plane, every row."""
    c, codes, lut, oc, ol = lm_head
    tiled = qmv.qtile_km4(codes)
    T = (oc.shape[0] + 63) // 64
    want_t = oc.reshape(T, 64, -1, 16).transpose(0, 2, 1, 3).reshape(-1)   # 248320 rows: whole tiles
    assert np.array_equal(host(tiled), want_t)
    y = host(qmv.qmatvec_km4_tiled(tiled, lut, dev(c.x[:1])))
    assert rel_err(y, oracle.matvec("km4", oc, ol, c.x[:1])) <= RTOL


def test_int8_head_full_and_high_rows():
    c = wl.int8_head()
    codes, scale = oracle.pack_int8(c.W)
    gc, gs = qmv.qpack_int8(dev(c.W))
    assert np.array_equal(codes, host(gc)) and np.array_equal(scale, host(gs))
    y = host(qmv.qmatvec_int8(gc, gs, dev(c.x)))[0]
    want = oracle.matvec("int8", codes, scale, c.x)[0]
    assert rel_err(y, want) <= RTOL
    # rows from 65024 up must be live wherever the reference is nonzero
    hi = np.arange(65024, c.W.shape[0])
    live = want[hi] != 0
    assert live.sum() > 0.99 * len(hi)
    assert np.all(y[hi][live] != 0)
    assert np.max(np.abs(y[hi] - want[hi])) <= RTOL * np.max(np.abs(want))


@pytest.fixture(scope="module")
def moe_case():
    c = wl.moe()
    E, I2, H = c.W_gate_up.shape
    I = I2 // 2
    gu = dev(c.W_gate_up.reshape(E * I2, H))
    dn = dev(c.W_down.reshape(E * H, I))
    guc, gus = qmv.qpack_int4(gu)
    dnc, dns = qmv.qpack_int4(dn)
    del gu, dn
    return c, guc.view(E, I2, H // 2), gus.view(E, I2, H // 32), dnc.view(E, H, I // 2), dns.view(E, H, I // 32)


def _oracle_experts(c, experts):
    """Oracle-packed slabs for the listed experts (others left zero)."""
    E, I2, H = c.W_gate_up.shape
    I = I2 // 2
    guc = np.zeros((E, I2, H // 2), np.uint8)
    gus = np.zeros((E, I2, H // 32), np.uint16)
    dnc = np.zeros((E, H, I // 2), np.uint8)
    dns = np.zeros((E, H, I // 32), np.uint16)
    for e in experts:
        guc[e], gus[e] = oracle.pack_int4(c.W_gate_up[e])
        dnc[e], dns[e] = oracle.pack_int4(c.W_down[e])
    return guc, gus, dnc, dns


def test_moe_route_parity(moe_case):
    c = moe_case[0]
    ids, w = qmv.qmoe_route(dev(c.logits), c.topk)
    oids, ow = oracle.moe_route(c.logits, c.topk)
    assert np.array_equal(host(ids), oids)
    assert np.allclose(host(w), ow, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_moe_layer_parity(moe_case, T):
    c, guc, gus, dnc, dns = moe_case
    logits, x = c.logits[:T], c.x[:T]
    oids, ow = oracle.moe_route(logits, c.topk)
    experts = np.unique(oids)
    ogu, ogs, odc, ods = _oracle_experts(c, experts)
    for e in experts:   # the GPU packed the routed experts bit-exactly
        assert np.array_equal(ogu[e], host(guc[e])) and np.array_equal(ogs[e], host(gus[e]))
        assert np.array_equal(odc[e], host(dnc[e])) and np.array_equal(ods[e], host(dns[e]))
    want, h_want = oracle.moe_ffn(ogu, ogs, odc, ods, x, oids, ow, return_h=True)
    y, ids, w = qmv.moe_ffn(guc, gus, dnc, dns, dev(x), dev(logits), c.topk)
    assert np.array_equal(host(ids), oids)
    assert rel_err(host(y), want) <= RTOL
    # the fused SwiGLU activations agree to within one fp16 step
    h = host(qmv.gather_qmatvec("int4", guc, gus, dev(x), ids, epi="swiglu")).astype(np.float64)
    step = np.abs(h_want) * 2.0 ** -10 + 2.0 ** -24
    assert np.all(np.abs(h - h_want) <= step)


def test_moe_gather_none_matches_per_slot_matvec(moe_case):
    c, guc, gus, dnc, dns = moe_case
    T = 3
    oids, _ = oracle.moe_route(c.logits[:T], c.topk)
    xs = np.random.default_rng(1).standard_normal((T, c.topk, 512)).astype(np.float16)
    y = host(qmv.gather_qmatvec("int4", dnc, dns, dev(xs), dev(oids), epi="none", x_per_slot=True))
    for t in range(T):
        for s in range(c.topk):
            e = oids[t, s]
            oc, os_ = oracle.pack_int4(c.W_down[e])
            want = oracle.matvec("int4", oc, os_, xs[t, s][None])[0]
            assert rel_err(y[t, s], want) <= RTOL


def test_moe_layer_replays_identically_in_a_hip_graph(moe_case):
    """The MoE entry points allocate nothing and never synchronize, so a layer
    can be captured in a HIP graph; every replay (with eager work between
    replays) must equal the eager result bit for bit."""
    import torch
    c, guc, gus, dnc, dns = moe_case
    T = 4
    E, H, I = guc.shape[0], 2 * guc.shape[2], guc.shape[1] // 2
    lg = dev(c.logits[:T])
    x = dev(c.x[:T])
    ids = torch.empty((T, c.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, c.topk), dtype=torch.float32, device="cuda")
    h = torch.empty((T, c.topk, I), dtype=torch.float16, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty((qmv.gather_qmatvec_workspace_bytes(T, c.topk, E, H, "combine"),), dtype=torch.uint8,
                     device="cuda")

    def layer():
        qmv.qmoe_route(lg, c.topk, ids=ids, weights=w)
        qmv.gather_qmatvec("int4", guc, gus, x, ids, epi="swiglu", y=h)
        qmv.gather_qmatvec("int4", dnc, dns, h, ids, weights=w, epi="combine", x_per_slot=True, y=y, workspace=ws)

    layer()
    torch.cuda.synchronize()
    ref = host(y).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for r in range(4):
        y.fill_(-1.0)
        ids.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), ref), "replay %d" % r
        layer()                      # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(host(y), ref)
