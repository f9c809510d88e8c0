"""The allocation-free fused argmax (qmatvec_argmax_noalloc) against the
workspace entry point (qmatvec_argmax): the same kernels, so the same row and
the same value bit for bit, on consecutive calls that reuse the library's
fixed device array with different sizes."""
import ctypes

import numpy as np
import pytest

import quantized_decode_matvec_amd as qmv

E_WORKSPACE = 5


def test_noalloc_refuses_sizes_beyond_its_array():
    L = qmv.lib()
    fake = ctypes.c_void_p(0x10000)            # never dereferenced: refused before any launch
    cap = int(L.qmatvec_argmax_noalloc_max_bytes())
    assert cap == 16 << 20
    assert int(L.qmatvec_argmax_workspace_bytes(248320, 8)) <= cap
    too_many_rows = (cap // 4) // 8 + 1        # y [8][N] fp32 alone exceeds the array
    st = L.qmatvec_argmax_noalloc(qmv.QMV_KM4, fake, fake, too_many_rows, 2048, fake, 8, fake, fake,
                                  ctypes.c_void_p(0))
    assert st == E_WORKSPACE
    assert b"workspace" in L.qmv_status_string(st)


def _case(torch, N, K, B, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    codes = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    lut = (torch.randn((N, 16), device="cuda", generator=g) * 0.02).sort(dim=1).values.half()
    x = torch.randn((B, K), device="cuda", generator=g).half()
    return codes, lut.view(torch.uint16), x


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    import torch
    cases = [(248320, 2048, 8, 1), (5000, 1024, 3, 2), (248320, 2048, 1, 3)]   # large, then smaller, then B = 1
    for N, K, B, seed in cases:
        print("noalloc case N=%d K=%d B=%d" % (N, K, B), flush=True)
        codes, lut, x = _case(torch, N, K, B, seed)
        i_ws, v_ws = qmv.qmatvec_argmax("km4", codes, lut, x)
        i_na, v_na = qmv.qmatvec_argmax_noalloc("km4", codes, lut, x)
        y = qmv.qmatvec_km4(codes, lut, x)
        torch.cuda.synchronize()
        i_ws, v_ws, i_na, v_na = (t.cpu().numpy() for t in (i_ws, v_ws, i_na, v_na))
        assert np.array_equal(i_na, i_ws) and np.array_equal(v_na.view(np.uint32), v_ws.view(np.uint32))
        yh = y.cpu().numpy()
        for b in range(B):
            assert v_na[b] == yh[b].max()
            assert i_na[b] == int(np.flatnonzero(yh[b] == yh[b].max())[0])    # lowest row among equals
