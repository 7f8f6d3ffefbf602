"""Pins of the fp64 oracle against things other than itself.

* central finite differences of L = sum(O * dO) (forward -> every gradient);
* torch's scaled_dot_product_attention + autograd in fp64 (a library routine),
  with GQA as repeated K/V and the sink reduced to one extra always-visible key;
* invariants of the softmax backward (rowsum of dS, sums of dV and dK);
* the GQA == MHA-with-repeated-K/V identity;
* closed forms (length-1 sequences, Q = 0) and special cases (sink -> -inf,
  window >= length, sequence independence of varlen packing).
"""
import numpy as np
import pytest
import torch

from oracle import attention as orc

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(lengths, hq, hkv, d, causal, window, sink, seed=0, qscale=1.0):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    t = int(cu[-1])
    return dict(
        q=rng.standard_normal((t, hq, d)) * qscale,
        k=rng.standard_normal((t, hkv, d)),
        v=rng.standard_normal((t, hkv, d)),
        do=rng.standard_normal((t, hq, d)),
        sink=rng.standard_normal(hq) if sink else None,
        cu_seqlens=cu, causal=causal, window=window, scale=1.0 / np.sqrt(d),
    )


MASKS = [(False, 0), (True, 0), (True, 3)]


def _loss(inp, q, k, v, sink):
    O, _ = orc.forward(q, k, v, inp["cu_seqlens"], inp["causal"], inp["window"], inp["scale"],
                       sink=sink)
    return float((O * inp["do"]).sum())


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("sink", [False, True])
def test_finite_differences(causal, window, sink):
    inp = _case([4, 6], 4, 2, 6, causal, window, sink, seed=1)
    g = orc.forward_backward(inp)
    eps = 1e-6
    for name, grad in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"]), ("sink", g["dsink"])):
        if inp[name] is None:
            continue
        x = inp[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {n: inp[n] for n in ("q", "k", "v", "sink")}
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args[name] = xp
            lp = _loss(inp, **args)
            args[name] = xm
            lm = _loss(inp, **args)
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.abs(fd - grad).max()
        assert err <= 1e-7 * max(1.0, np.abs(grad).max()), (name, err)


def _sdpa_reference(inp):
    """fp64 torch SDPA + autograd, per sequence, GQA via repeated K/V,
    sink as an extra key (q gets a trailing 1, the sink key is
    (0,...,0, sink/scale), its value vector is 0)."""
    q = torch.tensor(inp["q"], dtype=torch.float64)
    k = torch.tensor(inp["k"], dtype=torch.float64)
    v = torch.tensor(inp["v"], dtype=torch.float64)
    do = torch.tensor(inp["do"], dtype=torch.float64)
    sink = None if inp["sink"] is None else torch.tensor(inp["sink"], dtype=torch.float64,
                                                         requires_grad=True)
    q.requires_grad_(); k.requires_grad_(); v.requires_grad_()
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    scale = inp["scale"]
    outs = []
    cu = inp["cu_seqlens"]
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        qs = q[a:b].transpose(0, 1)  # [Hq, L, D]
        ks = k[a:b].repeat_interleave(G, dim=1).transpose(0, 1)
        vs = v[a:b].repeat_interleave(G, dim=1).transpose(0, 1)
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        mask = torch.ones(L, L, dtype=torch.bool)
        if inp["causal"]:
            mask &= j <= i
        if inp["window"]:
            mask &= j > i - inp["window"]
        mask = mask[None].expand(Hq, L, L)
        if sink is not None:
            qs = torch.cat([qs, torch.ones(Hq, L, 1, dtype=torch.float64)], dim=2)
            ks = torch.cat([ks, torch.zeros(Hq, L, 1, dtype=torch.float64)], dim=2)
            ksink = torch.cat([torch.zeros(Hq, 1, D, dtype=torch.float64),
                               (sink / scale)[:, None, None]], dim=2)
            ks = torch.cat([ks, ksink], dim=1)
            vs = torch.cat([vs, torch.zeros(Hq, 1, D, dtype=torch.float64)], dim=1)
            mask = torch.cat([mask, torch.ones(Hq, L, 1, dtype=torch.bool)], dim=2)
        o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask,
                                                             scale=scale)
        outs.append(o.transpose(0, 1))
    O = torch.cat(outs, dim=0)
    (O * do).sum().backward()
    return dict(o=O.detach().numpy(), dq=q.grad.numpy(), dk=k.grad.numpy(), dv=v.grad.numpy(),
                dsink=None if sink is None else sink.grad.numpy())


@pytest.mark.parametrize("causal,window", MASKS + [(True, 1)])
@pytest.mark.parametrize("sink", [False, True])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 4), (8, 1)])
def test_against_torch_sdpa(causal, window, sink, hq, hkv):
    inp = _case([9, 1, 14], hq, hkv, 8, causal, window, sink, seed=2)
    ref = _sdpa_reference(inp)
    got = orc.forward_backward(inp)
    for n in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(got[n], ref[n], rtol=0, atol=1e-12, err_msg=n)
    if sink:
        np.testing.assert_allclose(got["dsink"], ref["dsink"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("sink", [False, True])
def test_invariants(causal, window, sink):
    inp = _case([7, 12], 6, 2, 5, causal, window, sink, seed=3)
    g = orc.forward_backward(inp)
    G = 3
    cu = inp["cu_seqlens"]
    psink = (np.zeros_like(g["lse"]) if not sink
             else np.exp(inp["sink"][:, None] - g["lse"]))  # [Hq, T]
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for gg in range(2):
            hs = range(gg * G, (gg + 1) * G)
            # sum_j dV_j = sum_{h in g} sum_i (1 - p_sink_i) dO_i
            lhs = g["dv"][a:b, gg].sum(0)
            rhs = sum(((1 - psink[h, a:b])[:, None] * inp["do"][a:b, h]).sum(0) for h in hs)
            np.testing.assert_allclose(lhs, rhs, atol=1e-12)
            # sum_j dK_j = scale sum_{h in g} sum_i p_sink_i Delta_i q_i   (0 without sink)
            lhs = g["dk"][a:b, gg].sum(0)
            rhs = sum(inp["scale"] * ((psink[h, a:b] * g["delta"][h, a:b])[:, None]
                                      * inp["q"][a:b, h]).sum(0) for h in hs)
            np.testing.assert_allclose(lhs, rhs, atol=1e-12)
    if not sink:
        # rows of P sum to one without a sink, so sum_j dV_j = sum_i dO_i
        # (per sequence and group)
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            np.testing.assert_allclose(g["dv"][a:b].sum(axis=(0, 1)),
                                       inp["do"][a:b].sum(axis=(0, 1)), atol=1e-12)


def test_gqa_equals_repeated_mha():
    inp = _case([6, 9], 8, 2, 4, True, 4, True, seed=4)
    g = orc.forward_backward(inp)
    rep = dict(inp)
    rep["k"] = np.repeat(inp["k"], 4, axis=1)
    rep["v"] = np.repeat(inp["v"], 4, axis=1)
    m = orc.forward_backward(rep)
    np.testing.assert_array_equal(g["dq"], m["dq"])
    np.testing.assert_array_equal(g["o"], m["o"])
    np.testing.assert_allclose(g["dk"], m["dk"].reshape(-1, 2, 4, 4).sum(2), atol=1e-14)
    np.testing.assert_allclose(g["dv"], m["dv"].reshape(-1, 2, 4, 4).sum(2), atol=1e-14)
    np.testing.assert_allclose(g["dsink"], m["dsink"], atol=1e-14)


def test_length_one_sequences_closed_form():
    inp = _case([1, 1, 1], 4, 2, 8, True, 0, False, seed=5)
    g = orc.forward_backward(inp)
    for t in range(3):
        for h in range(4):
            np.testing.assert_allclose(g["o"][t, h], inp["v"][t, h // 2], atol=1e-15)
            assert abs(g["lse"][h, t] - inp["scale"] * inp["q"][t, h] @ inp["k"][t, h // 2]) < 1e-14
        for gg in range(2):
            np.testing.assert_allclose(g["dv"][t, gg], inp["do"][t, 2 * gg:2 * gg + 2].sum(0),
                                       atol=1e-15)
    assert np.abs(g["dq"]).max() < 1e-15 and np.abs(g["dk"]).max() < 1e-15


@pytest.mark.parametrize("causal,window", MASKS)
def test_zero_queries_closed_form(causal, window):
    inp = _case([5, 8], 2, 1, 3, causal, window, False, seed=6, qscale=0.0)
    g = orc.forward_backward(inp)
    cu = inp["cu_seqlens"]
    sc = inp["scale"]
    assert np.abs(g["dk"]).max() == 0.0
    for s in range(2):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        for h in range(2):
            for i in range(L):
                js = [j for j in range(L)
                      if (not causal or j <= i) and (window == 0 or j > i - window)]
                n = len(js)
                o = sum(inp["v"][a + j, 0] for j in js) / n
                np.testing.assert_allclose(g["o"][a + i, h], o, atol=1e-14)
                dlt = inp["do"][a + i, h] @ o
                dq = sum(sc * (inp["do"][a + i, h] @ inp["v"][a + j, 0] - dlt) / n
                         * inp["k"][a + j, 0] for j in js)
                np.testing.assert_allclose(g["dq"][a + i, h], dq, atol=1e-14)


def test_sink_to_minus_infinity_is_no_sink():
    a = _case([5, 7], 4, 2, 6, True, 3, True, seed=7)
    a["sink"] = np.full(4, -1e4)
    b = dict(a)
    b["sink"] = None
    ga, gb = orc.forward_backward(a), orc.forward_backward(b)
    for n in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(ga[n], gb[n])
    assert np.abs(ga["dsink"]).max() == 0.0


def test_window_at_least_length_is_causal():
    a = _case([6, 9], 4, 2, 5, True, 9, True, seed=8)
    b = dict(a)
    b["window"] = 0
    ga, gb = orc.forward_backward(a), orc.forward_backward(b)
    for n in ("o", "lse", "dq", "dk", "dv", "dsink"):
        np.testing.assert_allclose(ga[n], gb[n], atol=1e-15)


def test_window_counts():
    m = orc.visible(np.arange(10), np.arange(10), True, 4)
    assert list(m.sum(1)) == [min(i + 1, 4) for i in range(10)]
    assert m[9, 6] and not m[9, 5] and not m[3, 4]
    with pytest.raises(ValueError):
        orc.forward(np.zeros((2, 1, 2)), np.zeros((2, 1, 2)), np.zeros((2, 1, 2)), [0, 2],
                    False, 3, 1.0)


def test_varlen_sequences_are_independent():
    inp = _case([5, 8, 3], 4, 2, 4, True, 0, True, seed=9)
    g = orc.forward_backward(inp)
    cu = inp["cu_seqlens"]
    dsink = np.zeros(4)
    for s in range(3):
        a, b = int(cu[s]), int(cu[s + 1])
        one = {n: (inp[n][a:b] if n in ("q", "k", "v", "do") else inp[n]) for n in inp}
        one["cu_seqlens"] = np.array([0, b - a])
        gs = orc.forward_backward(one)
        for n in ("o", "dq", "dk", "dv"):
            np.testing.assert_allclose(g[n][a:b], gs[n], atol=1e-15)
        dsink += gs["dsink"]
    np.testing.assert_allclose(g["dsink"], dsink, atol=1e-14)


def test_row_chunking_does_not_change_results():
    inp = _case([23, 17], 4, 2, 8, True, 5, True, seed=10)
    a = orc.forward_backward(inp, row_chunk=4)
    b = orc.forward_backward(inp, row_chunk=1000)
    for n in ("o", "lse", "dq", "dk", "dv", "dsink"):
        np.testing.assert_allclose(a[n], b[n], atol=1e-13)


@pytest.mark.parametrize("causal,window,sink", [(False, 0, False), (True, 0, True), (True, 5, True)])
def test_sampled_rows_match_full(causal, window, sink):
    inp = _case([21, 13], 4, 2, 8, causal, window, sink, seed=11)
    g = orc.forward_backward(inp)
    rows = [(0, 0), (5, 3), (20, 1), (21, 2), (33, 3)]
    r = orc.query_rows(inp, rows)
    for n, (t, h) in enumerate(rows):
        np.testing.assert_allclose(r["o"][n], g["o"][t, h], atol=1e-14)
        np.testing.assert_allclose(r["dq"][n], g["dq"][t, h], atol=1e-14)
        assert abs(r["lse"][n] - g["lse"][h, t]) < 1e-13
        assert abs(r["delta"][n] - g["delta"][h, t]) < 1e-13
    krows = [(0, 0), (7, 1), (20, 0), (21, 1), (33, 0)]
    kr = orc.key_rows(inp, krows)
    for n, (t, gg) in enumerate(krows):
        np.testing.assert_allclose(kr["dk"][n], g["dk"][t, gg], atol=1e-13)
        np.testing.assert_allclose(kr["dv"][n], g["dv"][t, gg], atol=1e-13)
