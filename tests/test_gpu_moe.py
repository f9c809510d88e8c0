"""GPU parity of the mixture-of-experts entry points in every weight format,
on small expert sets that the oracle runs whole.

Cases cover one token (routing fused into the gate/up launch) and several,
one or several row tiles, ragged rows (96 = three 32-blocks), long gate/up
rows (4096) and long down rows (2048), and expert counts past 256 and 1024
(the wider routing layouts). Weights are packed by the oracle
and uploaded, so these tests see the MoE kernels alone; the packers have
their own bit-exact tests."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from tests.gpu_helpers import RTOL, dev, host, rel_err

pytestmark = pytest.mark.gpu

FORMATS = ["int4", "fp4", "int8", "km4", "int4aff", "int8km"]
# E, H, I, T, topk
CASES = [
    (16, 256, 128, 1, 3),
    (16, 256, 128, 5, 3),
    (300, 64, 32, 1, 8),
    (1500, 64, 32, 1, 8),
    (8, 96, 96, 8, 4),
    (4, 4096, 64, 3, 2),
    (6, 64, 2048, 2, 2),
    (300, 64, 32, 4, 8),
    (1500, 64, 32, 2, 8),
    # one token at hidden sizes 1280..2048 (several slots, the down rows of
    # 16 and 32 lanes)
    (10, 2048, 512, 1, 8),
    (12, 1536, 256, 1, 6),
    (8, 1280, 1024, 1, 4),
    # the down projection's two combine kernels: slot-split (topk <= 8, rows of
    # one chunk per lane, 8 or 16 rows per workgroup by token count, ragged row
    # tiles) and token-major (more slots, or longer rows)
    (16, 224, 64, 3, 8),
    (32, 256, 128, 3, 12),
    (4, 96, 4096, 2, 3),
]


def _case(fmt, E, H, I, T, topk, seed=0):
    rng = np.random.default_rng(seed + 7 * E + H + I)
    gu = (rng.standard_normal((E * 2 * I, H)) * 0.02).astype(np.float16)
    dn = (rng.standard_normal((E * H, I)) * 0.02).astype(np.float16)
    x = rng.standard_normal((T, H)).astype(np.float16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    guc, gup = oracle.pack(fmt, gu)
    dnc, dnp = oracle.pack(fmt, dn)
    guc, gup = guc.reshape(E, 2 * I, -1), gup.reshape(E, 2 * I, -1)
    dnc, dnp = dnc.reshape(E, H, -1), dnp.reshape(E, H, -1)
    return guc, gup, dnc, dnp, x, logits


def _h_close(h, h_want):
    """fp16 activations: within one fp16 step of the oracle's, plus the fp32
    accumulation error of the gate/up sums (1e-6 of the largest value)."""
    h = np.asarray(h, np.float64)
    tol = np.abs(h_want) * 2.0 ** -10 + 2.0 ** -24 + 1e-6 * np.abs(h_want).max()
    return np.all(np.abs(h - h_want) <= tol)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("E,H,I,T,topk", CASES)
def test_moe_ffn_matches_oracle(fmt, E, H, I, T, topk):
    print("moe_ffn", fmt, E, H, I, T, topk, flush=True)
    guc, gup, dnc, dnp, x, logits = _case(fmt, E, H, I, T, topk)
    oids, ow = oracle.moe_route(logits, topk)
    want, h_want = oracle.moe_ffn(guc, gup, dnc, dnp, x, oids, ow, return_h=True, fmt=fmt)
    d = [dev(a) for a in (guc, gup, dnc, dnp)]
    y, ids, w, h = qmv.qmoe_ffn(fmt, *d, dev(x), dev(logits), topk)
    assert np.array_equal(host(ids), oids)
    assert np.allclose(host(w), ow, rtol=1e-6, atol=1e-7)
    assert _h_close(host(h), h_want)
    assert rel_err(host(y), want) <= RTOL
    # the three-call path (route, SwiGLU gather, combine gather) computes the
    # same arithmetic in the same order: identical bits
    y3, ids3, w3 = qmv.moe_ffn(*d, dev(x), dev(logits), topk, fmt=fmt)
    assert np.array_equal(host(ids3), host(ids))
    assert np.array_equal(host(w3), host(w))
    assert np.array_equal(host(y3), host(y))


@pytest.mark.parametrize("fmt", FORMATS)
def test_gather_none_and_combine_with_shared_input(fmt):
    """epi=none gives every slot's own matvec; combine with one input per
    token (x_per_slot = 0) is the weighted sum over the token's slots."""
    E, H, I, T, topk = 12, 160, 64, 6, 3
    guc, gup, dnc, dnp, x, logits = _case(fmt, E, H, I, T, topk, seed=3)
    oids, ow = oracle.moe_route(logits, topk)
    codes, plane = dev(guc), dev(gup)
    y = host(qmv.gather_qmatvec(fmt, codes, plane, dev(x), dev(oids), epi="none"))
    yc = host(qmv.gather_qmatvec(fmt, codes, plane, dev(x), dev(oids), weights=dev(ow.astype(np.float32)),
                                 epi="combine"))
    for t in range(T):
        acc = np.zeros(2 * I)
        for s in range(topk):
            e = oids[t, s]
            want = oracle.matvec(fmt, guc[e], gup[e], x[t][None])[0]
            assert rel_err(y[t, s], want) <= RTOL
            acc += np.float64(np.float32(ow[t, s])) * want
        assert rel_err(yc[t], acc) <= RTOL


@pytest.mark.parametrize("fmt", ["int4", "fp4", "int8", "km4", "int4aff"])
@pytest.mark.parametrize("K", [96, 1024])
def test_combine_on_ragged_rows(fmt, K):
    """The weighted combine over 100 rows (a partial last row tile for both
    combine kernels) at T = 1, 2 and 5 tokens and 3, 8 and 11 slots, with one
    input per slot and one per token: every output row against the oracle's
    per-slot matvecs summed in fp64."""
    E, N = 12, 100
    rng = np.random.default_rng(K)
    W = (rng.standard_normal((E * N, K)) * 0.02).astype(np.float16)
    codes, plane = oracle.pack(fmt, W)
    codes, plane = codes.reshape(E, N, -1), plane.reshape(E, N, -1)
    for T in (1, 2, 5):
        for topk in (3, 8, 11):
            ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32)
            w = rng.random((T, topk)).astype(np.float32)
            for per_slot in (False, True):
                x = rng.standard_normal((T, topk, K) if per_slot else (T, K)).astype(np.float16)
                y = host(qmv.gather_qmatvec(fmt, dev(codes), dev(plane), dev(x), dev(ids), weights=dev(w),
                                            epi="combine", x_per_slot=per_slot))
                for t in range(T):
                    acc = np.zeros(N)
                    for s in range(topk):
                        xs = x[t, s] if per_slot else x[t]
                        acc += np.float64(w[t, s]) * oracle.matvec(fmt, codes[ids[t, s]], plane[ids[t, s]], xs[None])[0]
                    assert rel_err(y[t], acc) <= RTOL, (fmt, K, T, topk, per_slot)


@pytest.mark.parametrize("E,T", [(256, 64), (300, 37), (1500, 5), (4096, 3)])
def test_route_wide(E, T):
    rng = np.random.default_rng(E + T)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, E // 3] = logits[0, E - 1] = logits[0].max() + 0.5   # a tie: lower id first
    ids, w = qmv.qmoe_route(dev(logits), 8)
    oids, ow = oracle.moe_route(logits, 8)
    assert np.array_equal(host(ids), oids)
    assert np.allclose(host(w), ow, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("epi", ["none", "swiglu", "combine"])
def test_gather_clamps_out_of_range_ids(epi):
    """ids below 0 or at least E read as 0 or E - 1: the same bits as the
    call with the clamped ids."""
    fmt, E, H, I, T, topk = "int4", 12, 160, 64, 4, 3
    guc, gup, dnc, dnp, x, logits = _case(fmt, E, H, I, T, topk, seed=9)
    oids, ow = oracle.moe_route(logits, topk)
    bad = oids.copy()
    bad[0, 0], bad[1, 2], bad[3, 1] = -7, E, E + 100
    good = np.clip(bad, 0, E - 1).astype(np.int32)
    w = dev(ow.astype(np.float32)) if epi == "combine" else None
    codes, plane = dev(guc), dev(gup)
    yb = host(qmv.gather_qmatvec(fmt, codes, plane, dev(x), dev(bad.astype(np.int32)), weights=w, epi=epi))
    yg = host(qmv.gather_qmatvec(fmt, codes, plane, dev(x), dev(good), weights=w, epi=epi))
    assert np.array_equal(yb, yg)


def test_route_nan_logits_rank_last():
    """NaN logits rank below every number: ids stay valid and distinct and equal
    the oracle's on the logits with NaN replaced by -inf (there equal logits go
    to the lower id, as the NaN entries do here); one token has fewer finite
    logits than topk."""
    rng = np.random.default_rng(21)
    T, E, topk = 3, 256, 8
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, rng.choice(E, 5, replace=False)] = np.nan
    logits[1, :] = np.nan
    logits[1, rng.choice(E, 6, replace=False)] = rng.standard_normal(6).astype(np.float32)
    ids, w = qmv.qmoe_route(dev(logits), topk)
    ids, w = host(ids), host(w)
    oids, ow = oracle.moe_route(np.where(np.isnan(logits), -np.inf, logits).astype(np.float32), topk)
    assert np.array_equal(ids, oids)
    for t in range(T):
        assert len(set(ids[t].tolist())) == topk and ids[t].min() >= 0 and ids[t].max() < E
    assert np.allclose(w, ow, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("T,E,H,I,topk", [(1, 16, 256, 128, 3), (4, 16, 256, 128, 3), (1, 10, 2048, 512, 8)])
def test_moe_ffn_replays_identically_in_a_hip_graph(T, E, H, I, topk):
    """qmoe_ffn allocates nothing and never synchronizes, so it can be
    captured; each replay (with eager work between) equals the eager call."""
    import torch
    fmt = "km4"
    guc, gup, dnc, dnp, x, logits = _case(fmt, E, H, I, T, topk, seed=5)
    d = [dev(a) for a in (guc, gup, dnc, dnp)]
    xd, ld = dev(x), dev(logits)
    ids = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    h = torch.empty((T, topk, I), dtype=torch.float16, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def layer():
        qmv.qmoe_ffn(fmt, *d, xd, ld, topk, ids=ids, weights=w, h=h, y=y)

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
        layer()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), ref)
