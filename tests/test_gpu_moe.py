"""Parity of the grouped mixture-of-experts feed-forward with the oracle.

Routing (binary64 softmax, top-k, ties to the lower id) is computed once by
the oracle on the host and passed to both sides, so they route identically.
The check runs in stages, each against the oracle applied to the GPU's own
inputs to that stage:
  (i)   grouping: every assignment sits at a stable, per-expert position;
  (ii)  h (binary16, in the workspace) against silu(g)*u of the oracle, with a
        bound propagated from 2e-3 * S_g and 2e-3 * S_u plus binary16 rounding;
  (iii) d (binary32, in the workspace) against Wd_e h_gpu, bound 2e-3 * S_d;
  (iv)  out against sum_s w_s * (Wd_e h_gpu), bound 2e-3 * sum_s w_s S_d.
The end-to-end difference from the all-binary64 oracle is reported.
"""
import numpy as np
import pytest

import oracle
from quantized_unpack_q4_amd import gq, synth
from tests._gpu import dev, half_bits, host, say, torch_cuda, within

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _dsilu(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def _setup(seed, T, H, I, E, k, fmt=oracle.Q4_K):
    blocks = synth.q8_0_blocks if fmt == oracle.Q8_0 else synth.q4k_blocks
    wg = blocks(seed, 0, E * I, H)
    wu = blocks(seed, 1, E * I, H)
    wd = blocks(seed, 2, E * H, I)
    x16 = synth.activations_f16(seed, 0, T, H)
    ids, wts64 = oracle.moe_route(synth.router_logits(seed, 0, T, E), k)
    return wg, wu, wd, x16, ids, wts64.astype(np.float32)


def _run(wg, wu, wd, x16, ids, wts, H, I, E, input_weighted=False, fmt=oracle.Q4_K):
    out, ws = gq.moe_q4k(dev(wg), dev(wu), dev(wd), dev(x16), dev(ids), dev(wts), H, I, E,
                         input_weighted=input_weighted, q8_0=fmt == oracle.Q8_0)
    T, k = ids.shape
    off = gq.gq_moe_workspace_offsets(T, H, I, E, k)
    wsh = host(ws)
    A = T * k
    table = wsh[off[0]:off[0] + 4 * (E + 3)].view(np.int32)
    sorted_ = wsh[off[1]:off[1] + 4 * A].view(np.int32)
    pos_of = wsh[off[2]:off[2] + 4 * A].view(np.int32)
    h = wsh[off[4]:off[4] + 2 * A * I].view(np.float16).reshape(A, I)
    d = wsh[off[5]:off[5] + 4 * A * H].view(np.float32).reshape(A, H)
    o = half_bits(out).view(np.float16).astype(np.float64)
    return o, table, sorted_, pos_of, h, d


def _check_grouping(ids, E, table, sorted_, pos_of):
    T, k = ids.shape
    A = T * k
    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(table[:E], np.concatenate([[0], np.cumsum(counts)[:-1]]))
    assert table[E] == A and table[E + 2] == 0
    # stable order: sorted by (expert, assignment index)
    ref = np.lexsort((np.arange(A), flat))
    assert np.array_equal(sorted_, ref)
    assert np.array_equal(pos_of[sorted_], np.arange(A))


def _staged(wg, wu, wd, x16, ids, wts, H, I, E, o, table, sorted_, pos_of, h, d, toks,
            weight_input=False, fmt=oracle.Q4_K):
    """Stages (ii)-(iv).  weight_input: the slot weight w scales the expert's
    input, so stage (ii) expects silu(w g) * (w u) with the bounds of g and u
    scaled by w, and stage (iv) sums the slots' d unweighted."""
    T, k = ids.shape
    gu = I * oracle.row_bytes(fmt, H)
    dn = H * oracle.row_bytes(fmt, I)
    worst = {"h": 0.0, "d": 0.0, "out": 0.0}
    for t in toks:
        acc = np.zeros(H)
        accS = np.zeros(H)
        for s in range(k):
            a = t * k + s
            e = ids[t, s]
            p = pos_of[a]
            assert sorted_[p] == a
            # (ii) h against the oracle's g and u for this token and expert
            g, Sg = oracle.gemm(fmt, wg[e * gu:(e + 1) * gu], x16[t:t + 1], I, H)
            u, Su = oracle.gemm(fmt, wu[e * gu:(e + 1) * gu], x16[t:t + 1], I, H)
            g, Sg, u, Su = g[0], Sg[0], u[0], Su[0]
            if weight_input:
                pw = np.float64(wts[t, s])
                g, Sg, u, Su = pw * g, pw * Sg, pw * u, pw * Su
            href = _silu(g) * u
            bound = TOL * (np.abs(_dsilu(g) * u) * Sg + np.abs(_silu(g)) * Su) \
                + np.abs(href) * 2.0 ** -10 + 2.0 ** -24
            err = np.abs(h[p].astype(np.float64) - href)
            assert np.all(err <= bound), ("h", t, s, float((err - bound).max()))
            worst["h"] = max(worst["h"], float((err / bound).max()))
            # (iii) d against Wd_e applied to the GPU's own h
            dref, Sd = oracle.gemm(fmt, wd[e * dn:(e + 1) * dn],
                                   h[p:p + 1].view(np.uint16), H, I)
            worst["d"] = max(worst["d"], within(d[p], dref[0], Sd[0], TOL, "d"))
            wc = 1.0 if weight_input else np.float64(wts[t, s])
            acc += wc * dref[0]
            accS += wc * Sd[0]
        # (iv) combine
        worst["out"] = max(worst["out"], within(o[t], acc, accS, TOL, "out t=%d" % t))
    return worst


def test_moe_small_full():
    T, H, I, E, k = 5, 512, 256, 4, 2
    wg, wu, wd, x16, ids, wts = _setup(60, T, H, I, E, k)
    o, table, sorted_, pos_of, h, d = _run(wg, wu, wd, x16, ids, wts, H, I, E)
    _check_grouping(ids, E, table, sorted_, pos_of)
    worst = _staged(wg, wu, wd, x16, ids, wts, H, I, E, o, table, sorted_, pos_of, h, d,
                    range(T))
    r = oracle.moe_ffn(wg, wu, wd, x16, ids, wts, H, I, E)
    say("moe small staged", worst, "end-to-end", _e2e(o, r, wts))


def _e2e(o, r, wts):
    """Largest |out_gpu - out_ref| / sum_s w_s S_d over the binary64 oracle (reported)."""
    T, k = wts.shape
    Sd = r["Sd"].reshape(T, k, -1)
    bound = np.einsum("tk,tkh->th", np.abs(wts).astype(np.float64), Sd)
    return float((np.abs(o - r["out"]) / np.maximum(bound, 1e-300)).max())


def test_moe_empty_expert_and_dropped_ids():
    """Experts that receive no token, and ids outside [0, E), which are skipped."""
    T, H, I, E, k = 6, 256, 256, 8, 2
    wg, wu, wd, x16, _, _ = _setup(61, T, H, I, E, k)
    ids = np.array([[0, 3], [3, 0], [5, 3], [0, 5], [3, 9], [-1, 0]], np.int32)
    wts = np.full((T, k), 0.5, np.float32)
    o, table, sorted_, pos_of, h, d = _run(wg, wu, wd, x16, ids, wts, H, I, E)
    assert table[E + 2] == 2  # the two out-of-range ids
    assert pos_of[4 * 2 + 1] == -1 and pos_of[5 * 2 + 0] == -1
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E)
    assert np.array_equal(table[:E], np.concatenate([[0], np.cumsum(counts)[:-1]]))
    assert table[E] == valid.sum()
    # every valid slot still combines exactly like the full check
    ids_ok = np.where(valid, ids, 0)
    wts_ok = np.where(valid, wts, 0).astype(np.float32)
    r = oracle.moe_ffn(wg, wu, wd, x16, ids_ok, wts_ok, H, I, E)
    ratio = _e2e(o, r, wts_ok)
    say("moe dropped ids end-to-end", ratio)
    assert ratio <= 2 * TOL


def _staged_by_expert(wg, wu, wd, x16, ids, wts, H, I, E, o, sorted_, pos_of, h, d, toks,
                      fmt=oracle.Q4_K):
    """Stages (ii)-(iv) of _staged for many tokens, the oracle's products taken
    per expert over all of that expert's sampled assignments (its
    matrix-product form)."""
    T, k = ids.shape
    gu = I * oracle.row_bytes(fmt, H)
    dn = H * oracle.row_bytes(fmt, I)
    toks = np.asarray(sorted(set(int(t) for t in toks)))
    assign = np.array([t * k + s for t in toks for s in range(k)])
    dref = np.zeros((T * k, H))
    Sd = np.zeros((T * k, H))
    worst = {"h": 0.0, "d": 0.0, "out": 0.0}
    experts = ids.reshape(-1)
    for e in np.unique(experts[assign]):
        a_e = assign[experts[assign] == e]
        t_e = a_e // k
        p_e = pos_of[a_e]
        assert np.array_equal(sorted_[p_e], a_e)
        g, Sg = oracle.gemm_matmul(fmt, wg[e * gu:(e + 1) * gu], x16, I, H, toks=t_e)
        u, Su = oracle.gemm_matmul(fmt, wu[e * gu:(e + 1) * gu], x16, I, H, toks=t_e)
        href = _silu(g) * u
        bound = TOL * (np.abs(_dsilu(g) * u) * Sg + np.abs(_silu(g)) * Su) \
            + np.abs(href) * 2.0 ** -10 + 2.0 ** -24
        err = np.abs(h[p_e].astype(np.float64) - href)
        assert np.all(err <= bound), ("h", int(e), float((err - bound).max()))
        worst["h"] = max(worst["h"], float((err / bound).max()))
        dr, S = oracle.gemm_matmul(fmt, wd[e * dn:(e + 1) * dn], h[p_e].view(np.uint16), H, I)
        worst["d"] = max(worst["d"], within(d[p_e], dr, S, TOL, "d e=%d" % e))
        dref[a_e], Sd[a_e] = dr, S
    for t in toks:
        w_t = wts[t].astype(np.float64)
        acc = (w_t[:, None] * dref[t * k:(t + 1) * k]).sum(0)
        accS = (w_t[:, None] * Sd[t * k:(t + 1) * k]).sum(0)
        worst["out"] = max(worst["out"], within(o[t], acc, accS, TOL, "out t=%d" % t))
    return worst


def tokens_in_last_tiles(ids, E, n, g):
    """At least n tokens: for every expert, the token of its last assignment in
    the stable expert order (it sits in that expert's last, usually partial,
    token tile), then random tokens."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    last = {}
    for a in range(T * k):
        last[int(flat[a])] = a // k
    picked = set(last.values()) | {0, T - 1}
    rest = [t for t in g.permutation(T) if t not in picked]
    picked |= set(int(t) for t in rest[:max(0, n - len(picked))])
    return sorted(picked)


@pytest.mark.parametrize("T", [256, 2048])
def test_moe_olmoe_shape_sampled(T):
    """OLMoE-1B-7B-shaped layer (64 experts, top-8, hidden 2048, expert 1024) at
    full size; grouping checked whole, values on at least 64 tokens including
    every expert's last token (its ragged remainder tile)."""
    H, I, E, k = 2048, 1024, 64, 8
    say("moe olmoe T", T)
    wg, wu, wd, x16, ids, wts = _setup(4, T, H, I, E, k)
    o, table, sorted_, pos_of, h, d = _run(wg, wu, wd, x16, ids, wts, H, I, E)
    _check_grouping(ids, E, table, sorted_, pos_of)
    toks = tokens_in_last_tiles(ids, E, 96, np.random.default_rng(7))
    assert len(toks) >= 64
    say("  checking", len(toks), "tokens")
    worst = _staged_by_expert(wg, wu, wd, x16, ids, wts, H, I, E, o, sorted_, pos_of, h, d, toks)
    say("  staged worst ratios", worst)


def test_moe_few_tokens_per_expert_chunks():
    """Few tokens per expert on average (the weight-streaming path), with one
    expert over its 64-token chunk (80 tokens) and ragged counts elsewhere;
    every token checked in stages."""
    T, H, I, E, k = 100, 512, 256, 8, 2
    wg, wu, wd, x16, _, _ = _setup(62, T, H, I, E, k)
    ids = np.zeros((T, k), np.int32)
    for t in range(T):
        ids[t] = [0, 1 + t % 7] if t < 80 else [2 + t % 5, 7]
    g = np.random.default_rng(63)
    wts = g.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    o, table, sorted_, pos_of, h, d = _run(wg, wu, wd, x16, ids, wts, H, I, E)
    _check_grouping(ids, E, table, sorted_, pos_of)
    worst = _staged(wg, wu, wd, x16, ids, wts, H, I, E, o, table, sorted_, pos_of, h, d,
                    range(T))
    say("moe chunks staged", worst)


def test_moe_many_tokens_per_expert_tiles():
    """Many tokens per expert on average (the 256 x 256 tile path): an expert
    with more than one ragged 256-token tile, an expert with none, every token
    checked in stages."""
    T, H, I, E, k = 700, 512, 256, 8, 2
    wg, wu, wd, x16, _, _ = _setup(64, T, H, I, E, k)
    g = np.random.default_rng(65)
    ids = np.zeros((T, k), np.int32)
    for t in range(T):
        first = 0 if t < 380 else int(g.integers(1, 7))
        second = int(g.integers(1, 7))
        while second == first:
            second = int(g.integers(1, 7))
        ids[t] = [first, second]  # expert 7 gets nothing, expert 0 gets 380 tokens
    wts = g.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    o, table, sorted_, pos_of, h, d = _run(wg, wu, wd, x16, ids, wts, H, I, E)
    _check_grouping(ids, E, table, sorted_, pos_of)
    worst = _staged(wg, wu, wd, x16, ids, wts, H, I, E, o, table, sorted_, pos_of, h, d,
                    range(T))
    say("moe tiles staged", worst)


@pytest.mark.parametrize("T", [100, 300, 700])
def test_moe_input_weighted(T):
    """Slot weights applied to the experts' inputs (gq_moe_gemm_q4k_input_weighted)
    in each regime: 100, 300 and 700 tokens over 8 experts, top-2, are about
    25, 75 and 175 tokens per expert (weight streaming, 128-row tiles,
    256 x 256 tiles); grouping whole, values in stages on sampled tokens, and
    the end-to-end difference from the binary64 oracle of the same form."""
    H, I, E, k = 512, 256, 8, 2
    say("moe input weighted T", T)
    wg, wu, wd, x16, ids, wts = _setup(66, T, H, I, E, k)
    o, table, sorted_, pos_of, h, d = _run(wg, wu, wd, x16, ids, wts, H, I, E,
                                           input_weighted=True)
    _check_grouping(ids, E, table, sorted_, pos_of)
    toks = sorted(set([0, 1, T // 3, T // 2, T - 2, T - 1]))
    worst = _staged(wg, wu, wd, x16, ids, wts, H, I, E, o, table, sorted_, pos_of, h, d, toks,
                    weight_input=True)
    r = oracle.moe_ffn(wg, wu, wd, x16[toks], ids[toks], wts[toks], H, I, E, weight_input=True)
    bound = r["Sd"].reshape(len(toks), k, -1).sum(axis=1)
    e2e = float((np.abs(o[toks] - r["out"]) / np.maximum(bound, 1e-300)).max())
    say("  staged", worst, "end-to-end", e2e)


@pytest.mark.parametrize("T,weight_input", [(5, False), (100, False), (100, True), (300, False),
                                            (700, False), (300, True)])
def test_moe_q8_0(T, weight_input):
    """Q8_0 expert stacks (gq_moe_gemm_q8_0 and its input-weighted form): 100
    tokens over 8 experts, top-2 (25 per expert), stream the weights; 300
    takes the 64-token tiles of the 128-row kernel and 700 the 256 x 256
    tiles; 5 tokens over 4 experts checks every token."""
    E, k = (4, 2) if T == 5 else (8, 2)
    H, I = 512, 256
    say("moe q8_0 T", T, "input weighted", weight_input)
    wg, wu, wd, x16, ids, wts = _setup(67, T, H, I, E, k, fmt=oracle.Q8_0)
    o, table, sorted_, pos_of, h, d = _run(wg, wu, wd, x16, ids, wts, H, I, E,
                                           input_weighted=weight_input, fmt=oracle.Q8_0)
    _check_grouping(ids, E, table, sorted_, pos_of)
    toks = range(T) if T == 5 else sorted(set([0, 1, T // 3, T // 2, T - 2, T - 1]))
    toks = list(toks)
    worst = _staged(wg, wu, wd, x16, ids, wts, H, I, E, o, table, sorted_, pos_of, h, d, toks,
                    weight_input=weight_input, fmt=oracle.Q8_0)
    r = oracle.moe_ffn(wg, wu, wd, x16[toks], ids[toks], wts[toks], H, I, E,
                       weight_input=weight_input, fmt=oracle.Q8_0)
    wsum = np.ones_like(wts[toks]) if weight_input else wts[toks]
    say("  staged", worst, "end-to-end", _e2e(o[toks], r, wsum))


def test_moe_q8_0_many_tokens_per_expert_tiles():
    """Q8_0 stacks on the 256 x 256 tiles: an expert with a full tile and a
    44-token remainder (the reduced remainder tile), an expert with none,
    every token checked in stages and end to end."""
    T, H, I, E, k = 620, 512, 256, 8, 2
    wg, wu, wd, x16, _, _ = _setup(68, T, H, I, E, k, fmt=oracle.Q8_0)
    g = np.random.default_rng(69)
    ids = np.zeros((T, k), np.int32)
    for t in range(T):
        first = 0 if t < 300 else int(g.integers(1, 7))
        second = int(g.integers(1, 7))
        while second == first:
            second = int(g.integers(1, 7))
        ids[t] = [first, second]  # expert 7 gets nothing, expert 0 gets 256 + 44 tokens
    wts = g.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    o, table, sorted_, pos_of, h, d = _run(wg, wu, wd, x16, ids, wts, H, I, E, fmt=oracle.Q8_0)
    _check_grouping(ids, E, table, sorted_, pos_of)
    worst = _staged(wg, wu, wd, x16, ids, wts, H, I, E, o, table, sorted_, pos_of, h, d,
                    range(T), fmt=oracle.Q8_0)
    toks = list(range(0, T, 7))
    r = oracle.moe_ffn(wg, wu, wd, x16[toks], ids[toks], wts[toks], H, I, E, fmt=oracle.Q8_0)
    say("moe q8_0 tiles staged", worst, "end-to-end", _e2e(o[toks], r, wts[toks]))


@pytest.mark.parametrize("rows", [261, 2054])
def test_moe_expert_parallel_share(rows):
    """One GPU's expert-parallel share as the benchmark runs it: 8 experts,
    one dispatched row per (token, local expert) pair, top-1 routing with the
    slot's weight (261 rows stream the weights, 2054 take the large tiles);
    grouping whole, stages on sampled rows."""
    H, I, E, k = 2048, 1024, 8, 1
    say("moe ep share rows", rows)
    g = np.random.default_rng(rows)
    wg = synth.q4k_blocks(68, 0, E * I, H)
    wu = synth.q4k_blocks(68, 1, E * I, H)
    wd = synth.q4k_blocks(68, 2, E * H, I)
    x16 = synth.activations_f16(68, 0, rows, H)
    ids = g.integers(0, E, (rows, 1)).astype(np.int32)
    wts = g.uniform(0.02, 0.4, (rows, 1)).astype(np.float32)
    o, table, sorted_, pos_of, h, d = _run(wg, wu, wd, x16, ids, wts, H, I, E)
    _check_grouping(ids, E, table, sorted_, pos_of)
    toks = sorted(set([0, 1, rows // 3, rows // 2, rows - 2, rows - 1]))
    worst = _staged(wg, wu, wd, x16, ids, wts, H, I, E, o, table, sorted_, pos_of, h, d, toks)
    say("  staged", worst)
