"""Expert routing on the device (gq_moe_route) against the binary64 oracle.

Ids: bit-exact.  Softmax is strictly increasing, so the top-k experts are the
top-k logits; the kernel compares the binary32 logits exactly and the oracle
ranks binary64 probabilities computed from the same logits, which keep the
order of distinct logits and tie equal ones (for logits spanning less than
~700, where no probability underflows).  Equal logits go to the lower expert
index on both sides.

Weights: binary32 softmax against binary64.  Each probability is
exp(l - max) / sum: the subtraction rounds once (relative 2^-24 of |l - max|,
under 2^-20 in the exponent for the N(0,1) and integer logits here), expf is
within a few ulp, the sum of at most 256 positive terms over a butterfly adds
at most ~10 roundings, the division one: about 2e-6 relative in all, checked
against 1e-5 (renormalised weights: one more sum and division, same bound).
"""
import numpy as np
import pytest

import oracle
from quantized_unpack_q4_amd import gq, synth
from tests._gpu import dev, say, torch_cuda

pytestmark = pytest.mark.gpu

RTOL = 1e-5


def _route(logits, k, renorm):
    torch = torch_cuda()
    ids, wts = gq.moe_route(dev(logits), k, renormalize=renorm)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), wts.cpu().numpy().astype(np.float64)


def _check(logits, k, renorm, what):
    ids, wts = _route(logits, k, renorm)
    ids_r, wts_r = oracle.moe_route(logits, k, renormalize=renorm)
    assert np.array_equal(ids, ids_r), "%s: ids differ at %s" % (
        what, np.argwhere(ids != ids_r)[:5].tolist())
    err = np.abs(wts - wts_r) / np.maximum(wts_r, 1e-300)
    assert err.max() <= RTOL, "%s: weight error %.3g" % (what, err.max())
    return err.max()


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("T", [1, 7, 256, 2048])
def test_route_olmoe_shape(T, renorm):
    """64 experts, top-8, N(0,1) logits: the routing the mixture-of-experts
    layer uses, at 256 and 2048 tokens and ragged token counts."""
    say("route", T, renorm)
    logits = synth.router_logits(41, 0, T, 64)
    say("  max rel err", _check(logits, 8, renorm, "T=%d" % T))


@pytest.mark.parametrize("E,k", [(60, 1), (60, 60), (200, 8), (200, 65), (256, 256), (1, 1)])
def test_route_expert_counts(E, k):
    """Expert counts not a multiple of 64, top-1, top-k of all experts, and
    more than 64 slots (kept in a lane's second register)."""
    say("route E k", E, k)
    logits = synth.router_logits(42, E, 33, E)
    for renorm in (False, True):
        _check(logits, k, renorm, "E=%d k=%d renorm=%s" % (E, k, renorm))


def test_route_exact_ties_go_to_lower_index():
    """Integer logits with many exact ties, a row of all-equal logits and a
    duplicated maximum: equal logits must go to the lower expert index."""
    g = np.random.default_rng(43)
    logits = g.integers(-3, 4, size=(64, 64)).astype(np.float32)
    logits[0, :] = 0.25
    logits[1, 40] = logits[1, 7] = 9.0
    for renorm in (False, True):
        _check(logits, 8, renorm, "ties renorm=%s" % renorm)
    ids, _ = _route(logits, 8, False)
    assert list(ids[0]) == list(range(8)) and list(ids[1][:2]) == [7, 40]


def test_route_feeds_the_moe_layer():
    """Device routing gives the layer the same experts as host routing, and
    weights within the routing bound: the layer's outputs agree to its own
    binary16 tolerance."""
    torch = torch_cuda()
    T, H, I, E, k = 64, 512, 256, 16, 4
    wg = dev(synth.q4k_blocks(44, 0, E * I, H))
    wu = dev(synth.q4k_blocks(44, 1, E * I, H))
    wd = dev(synth.q4k_blocks(44, 2, E * H, I))
    x16 = dev(synth.activations_f16(44, 0, T, H))
    logits = synth.router_logits(44, 0, T, E)
    ids_h, wts_h = oracle.moe_route(logits, k)
    out_h, _ = gq.moe_q4k(wg, wu, wd, x16, dev(ids_h), dev(wts_h.astype(np.float32)), H, I, E)
    ids_d, wts_d = gq.moe_route(dev(logits), k)
    out_d, _ = gq.moe_q4k(wg, wu, wd, x16, ids_d, wts_d, H, I, E)
    torch.cuda.synchronize()
    assert np.array_equal(ids_d.cpu().numpy(), ids_h)
    a = out_h.float().cpu().numpy()
    b = out_d.float().cpu().numpy()
    assert np.all(np.abs(a - b) <= 2e-3 * np.abs(a) + 1e-3 * np.abs(a).max())
