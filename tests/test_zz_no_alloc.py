"""The allocation-free Fisher entry point (lrc_fisher_scores_noalloc, partials in the library's own
device scratch array) against lrc_fisher_scores (caller workspace) through the C ABI: bit-identical
scores on two calls in a row, the second with a smaller input, and a too-large input rejected on
the host before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

from activation_aware_rank_amd import inputs
from parity_utils import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lrc():
    from activation_aware_rank_amd import lrc as m
    return m


def _mats(shapes, seed):
    Gs, Ws = [], []
    for i, (r, c) in enumerate(shapes):
        Gs.append(dev(inputs.gradient(r, c, 1e-4, inputs.CFG_STACK, seed, i), "bf16"))
        Ws.append(dev(inputs.weight(r, c, "bf16", inputs.CFG_STACK, seed, i), "bf16"))
    return Gs, Ws


def _both(lrc, Gs, Ws):
    a_ref, i_ref = lrc.lrc_fisher_scores(Gs, Ws)
    n = len(Gs)
    alpha = torch.full((n,), -1.0, dtype=torch.float64, device="cuda")
    info = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    lrc.lrc_fisher_scores_noalloc(Gs, Ws, alpha, info)
    return host(a_ref), host(i_ref), host(alpha), host(info)


def test_noalloc_matches_workspace_entry_two_calls(lrc):
    print("\n[case] Fisher without allocation: 7 block-shaped matrices, then 3 small ones", flush=True)
    big = [(4096, 4096), (4096, 1024), (1024, 4096), (4096, 3000), (4096, 11008), (11008, 4096), (777, 333)]
    Gs, Ws = _mats(big, 0)
    a_ref, i_ref, a, i = _both(lrc, Gs, Ws)
    assert np.array_equal(a, a_ref) and np.array_equal(i, i_ref) and np.all(i == 0)
    small = [(100, 37), (64, 64), (1, 5)]
    Gs2, Ws2 = _mats(small, 1)
    a_ref2, i_ref2, a2, i2 = _both(lrc, Gs2, Ws2)
    assert np.array_equal(a2, a_ref2) and np.array_equal(i2, i_ref2) and np.all(i2 == 0)
    print("alpha %s / %s" % (a[:2], a2), flush=True)


def test_noalloc_rejects_input_beyond_the_scratch(lrc):
    """2^19 blocks of 32768 elements is the limit: one element more is rejected synchronously (the
    pointers are never dereferenced, nothing is launched)."""
    fake = ctypes.c_void_p(256)
    gp = (ctypes.c_void_p * 2)(fake, fake)
    ne = (ctypes.c_int64 * 2)((1 << 19) * 32768, 1)
    alpha = torch.zeros(2, dtype=torch.float64, device="cuda")
    info = torch.zeros(2, dtype=torch.int32, device="cuda")
    rc = lrc._fsh_na(2, gp, gp, ne, 0, ctypes.c_void_p(alpha.data_ptr()), ctypes.c_void_p(info.data_ptr()), None)
    assert rc == 1 and "scratch" in lrc.lrc_last_error()
