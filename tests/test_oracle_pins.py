"""Pins of the CPU oracle to facts other than itself.

Each test checks the oracle against one of: a hand-derived vector from the
pages (tests/golden, each with its citation), a brute-force computation on
tiny inputs written differently (pure-Python sorts and loops, a dense gating
formulation over every expert), a library routine (torch.softmax,
torch.nn.functional.silu, torch matmul), a closed form, or an invariant the
pages fix (zero-weight pairs contribute nothing; the identity slot table
equals expert-indexed compute; replicas are interchangeable; expert-parallel
partial outputs sum to the full output). The mutation tests at the end plant
plausible mistakes in the oracle and check that a pin catches each one.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.moe_oracle as om
from conftest import load_golden
from workloads import WorkloadConfig, build_slot_table, identity_slot_table, make_inputs, slot_weights

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- helpers
def py_topk(row, K):
    """Full pure-Python sort of all experts by (logit descending, id ascending)."""
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:K]


def dense_brute(x, logits, wgu, wd, K, renorm, ep_size=1, ep_rank=0, w_override=None,
                on_input=False):
    """Dense gating in torch fp64: every local expert on every token,
    out = sum_e G[t,e] * MLP_e(x_t), with G from a pure-Python full sort and
    torch.softmax; the MLP uses torch's silu and matmul. on_input: out =
    sum_e MLP_e(G[t,e] * x_t) (an unselected expert has G = 0 and, with no
    biases, MLP_e(0) = 0)."""
    x = torch.as_tensor(np.asarray(x, dtype=np.float64))
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    I = wd.shape[2]
    p = torch.softmax(torch.as_tensor(lg), dim=1)
    G = torch.zeros(T, E, dtype=torch.float64)
    for t in range(T):
        sel = py_topk(lg[t], K)
        ws = [float(p[t, e]) for e in sel]
        if w_override is not None:
            ws = [float(v) for v in w_override[t]]
        elif renorm:
            s = math.fsum(ws)
            ws = [v / s for v in ws]
        for e, v in zip(sel, ws):
            G[t, e] += v
    El = E // ep_size
    lo, hi = ep_rank * El, (ep_rank + 1) * El
    out = torch.zeros(T, x.shape[1], dtype=torch.float64)
    for e in range(lo, hi):
        w = torch.as_tensor(np.asarray(wgu[e], dtype=np.float64))
        d = torch.as_tensor(np.asarray(wd[e], dtype=np.float64))
        if on_input:
            xe = G[:, e:e + 1] * x
            out += (F.silu(xe @ w[:I].T) * (xe @ w[I:].T)) @ d.T
        else:
            g = x @ w[:I].T
            u = x @ w[I:].T
            out += G[:, e:e + 1] * ((F.silu(g) * u) @ d.T)
    return out.numpy()


def tiny_problem(seed, T=11, H=12, I=10, E=6, K=3, ties=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    lg = rng.standard_normal((T, E))
    if ties:
        lg = np.round(lg * 2) / 2  # few distinct values -> many ties
    wgu = rng.standard_normal((E, 2 * I, H)) / math.sqrt(H)
    wd = rng.standard_normal((E, H, I)) / math.sqrt(I)
    return x, lg.astype(np.float32), wgu, wd


# ---------------------------------------------------------------- route
def test_route_golden_vectors():
    g = load_golden("route_ties.json")
    for c in g["cases"]:
        ids, w = oracle.route(np.array(c["logits"], dtype=np.float32), c["K"], c["renormalize"])
        assert ids.tolist() == c["ids"]
        if c["w"] is not None:
            np.testing.assert_allclose(w, np.array(c["w"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("ties", [False, True])
def test_topk_matches_full_python_sort(seed, ties):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 40))
    K = int(rng.integers(1, E + 1))
    _, lg, _, _ = tiny_problem(seed, T=9, E=E, ties=ties)
    ids = oracle.topk_ids(lg, K)
    for t in range(lg.shape[0]):
        assert ids[t].tolist() == py_topk(lg[t], K)


def test_softmax_matches_torch():
    _, lg, _, _ = tiny_problem(3, T=20, E=33)
    ref = torch.softmax(torch.as_tensor(lg, dtype=torch.float64), dim=1).numpy()
    np.testing.assert_allclose(oracle.softmax(lg), ref, rtol=1e-14, atol=0)


def test_route_weights_closed_forms():
    _, lg, _, _ = tiny_problem(4, T=16, E=9)
    p = torch.softmax(torch.as_tensor(lg, dtype=torch.float64), dim=1).numpy()
    ids, w = oracle.route(lg, 4, False)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-14)
    _, wr = oracle.route(lg, 4, True)
    np.testing.assert_allclose(wr.sum(1), 1.0, rtol=0, atol=1e-15)
    # K = 1 with renormalisation: exactly 1.0 (x / x)
    _, w1 = oracle.route(lg, 1, True)
    assert (w1 == 1.0).all()
    # K = E: every expert once, weights = full softmax in sorted order
    ids_all, w_all = oracle.route(lg, 9, False)
    assert all(sorted(r) == list(range(9)) for r in ids_all.tolist())
    np.testing.assert_allclose(w_all.sum(1), 1.0, atol=1e-14)


def test_route_grouped_golden_vectors():
    for c in load_golden("route_grouped.json")["cases"]:
        logits = np.array([c["logits"]], dtype=np.float32)
        ids, w = oracle.route_grouped(logits, c["K"], False, c["num_groups"], c["topk_groups"])
        assert ids[0].tolist() == c["ids"], c["name"]
        p = oracle.softmax(logits)[0]
        np.testing.assert_array_equal(w[0], p[ids[0]])


def _grouped_bruteforce(l, K, G, TG):
    E = len(l)
    Eg = E // G
    groups = []
    for g in range(G):
        best = max(l[g * Eg:(g + 1) * Eg])
        groups.append((-best, g))
    groups.sort()
    cand = []
    for _, g in groups[:TG]:
        for e in range(g * Eg, (g + 1) * Eg):
            cand.append((-l[e], e))
    cand.sort()
    return [e for _, e in cand[:K]]


@pytest.mark.parametrize("seed", range(6))
def test_route_grouped_bruteforce(seed):
    rng = np.random.default_rng(200 + seed)
    E, G, TG, K = [(16, 4, 2, 3), (160, 8, 3, 6), (64, 8, 4, 8), (12, 3, 1, 4), (32, 32, 5, 5),
                   (8, 2, 2, 8)][seed]
    T = 20
    l = rng.standard_normal((T, E)).astype(np.float32)
    if seed % 2:
        l = np.round(l * 2) / 2  # many ties
    ids, w = oracle.route_grouped(l, K, True, G, TG)
    for t in range(T):
        assert ids[t].tolist() == _grouped_bruteforce(l[t].tolist(), K, G, TG)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-12)


@pytest.mark.parametrize("G,TG", [(1, 1), (4, 4), (8, 8)])
def test_route_grouped_reduces_to_plain_topk(G, TG):
    """One group, or every group kept: the grouping selects nothing away."""
    rng = np.random.default_rng(G)
    l = rng.standard_normal((30, 32)).astype(np.float32)
    for renorm in (False, True):
        a = oracle.route_grouped(l, 5, renorm, G, TG)
        b = oracle.route(l, 5, renorm)
        assert np.array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def test_mutation_grouped_sum_score_is_caught(monkeypatch):
    # planted mistake: a group scored by the sum of its logits instead of the max
    def bad(logits, K, renormalize, num_groups, topk_groups):
        l = np.asarray(logits, dtype=np.float64)
        T, E = l.shape
        Eg = E // num_groups
        gs = l.reshape(T, num_groups, Eg).sum(axis=2)
        ids = np.empty((T, K), dtype=np.int64)
        for t in range(T):
            order = np.lexsort((np.arange(num_groups), -gs[t]))[:topk_groups]
            keep = np.zeros(E, dtype=bool)
            for g in order:
                keep[g * Eg:(g + 1) * Eg] = True
            ids[t] = om.topk_ids(np.where(keep, l[t], -np.inf)[None, :], K)[0]
        return ids.astype(np.int32), np.take_along_axis(om.softmax(l), ids, axis=1)
    monkeypatch.setattr(om, "route_grouped", bad)
    monkeypatch.setattr(oracle, "route_grouped", bad)
    with pytest.raises(AssertionError):
        test_route_grouped_golden_vectors()


def test_route_all_equal_logits():
    lg = np.full((3, 7), 0.25, dtype=np.float32)
    ids, w = oracle.route(lg, 3, False)
    assert (ids == np.arange(3)).all()
    np.testing.assert_allclose(w, 1.0 / 7.0, rtol=1e-15)


# ---------------------------------------------------------------- slot map
def test_slot_map_golden_vectors():
    for c in load_golden("slot_map_ep.json")["cases"]:
        ro = None if c["rep_off"] is None else np.array(c["rep_off"])
        rs = None if c["rep_slots"] is None else np.array(c["rep_slots"])
        slot, wm, mask = oracle.slot_map(np.array(c["ids"]), np.array(c["w"]), c["E_global"],
                                         c["ep_size"], c["ep_rank"], ro, rs)
        assert slot.tolist() == c["slot"], c["name"]
        assert mask.tolist() == c["mask"], c["name"]
        np.testing.assert_array_equal(wm, np.array(c["w_masked"]))


@pytest.mark.parametrize("seed", range(4))
def test_slot_map_scalar_bruteforce(seed):
    rng = np.random.default_rng(seed)
    ep_size = int(rng.choice([1, 2, 3, 4]))
    El = int(rng.integers(1, 6))
    E = El * ep_size
    T, K = 13, min(3, E)
    ids = rng.integers(0, E, size=(T, K))
    w = rng.random((T, K))
    nrep = int(rng.integers(0, El + 1))
    reps = sorted(rng.choice(El, size=nrep, replace=False).tolist())
    ro, rs, slot_expert = build_slot_table(El, reps)
    for r in range(ep_size):
        slot, wm, mask = oracle.slot_map(ids, w, E, ep_size, r, ro.numpy(), rs.numpy())
        start = r * El
        for t in range(T):
            for k in range(K):
                e = int(ids[t, k])
                local = start <= e < start + El
                lid = e - start if local else e % El
                lst = [s for s in range(len(slot_expert)) if int(slot_expert[s]) == lid]
                assert mask[t, k] == int(local)
                assert wm[t, k] == (w[t, k] if local else 0.0)
                assert slot[t, k] == lst[t % len(lst)]


def test_slot_map_partition_invariants():
    rng = np.random.default_rng(7)
    E, ep = 12, 4
    ids = rng.integers(0, E, size=(50, 3))
    w = rng.random((50, 3))
    total = np.zeros(ids.shape, dtype=np.int64)
    for r in range(ep):
        slot, wm, mask = oracle.slot_map(ids, w, E, ep, r)
        assert ((slot >= 0) & (slot < E // ep)).all()
        total += mask
    assert (total == 1).all()  # every pair is local on exactly one rank
    slot, wm, mask = oracle.slot_map(ids, w, E, 1, 0)
    assert (mask == 1).all() and (slot == ids).all() and (wm == w).all()
    with pytest.raises(ValueError):
        oracle.slot_map(ids, w, 10, 4, 0)


# ---------------------------------------------------------------- permute
def test_permute_golden_vectors():
    for c in load_golden("permute_example.json")["cases"]:
        off, sp, pr = oracle.permute_indices(np.array(c["slot"]), np.array(c["mask"]), c["S"])
        assert off.tolist() == c["offsets"], c["name"]
        assert sp.tolist() == c["sorted_pairs"], c["name"]
        assert pr.tolist() == c["pair_row"], c["name"]


@pytest.mark.parametrize("seed", range(5))
def test_permute_bruteforce_and_invariants(seed):
    rng = np.random.default_rng(seed)
    T, K, S = int(rng.integers(0, 30)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
    slot = rng.integers(0, S, size=(T, K))
    mask = (rng.random((T, K)) < 0.7).astype(np.uint8)
    off, sp, pr = oracle.permute_indices(slot, mask, S)
    # brute force: for each slot in order, scan the pairs in order
    order = [p for s in range(S) for p in range(T * K)
             if mask.ravel()[p] and slot.ravel()[p] == s]
    assert sp.tolist() == order
    assert off[-1] == int(mask.sum()) and (np.diff(off) >= 0).all()
    for s in range(S):
        assert off[s + 1] - off[s] == int(((slot == s) & (mask == 1)).sum())
    rows = pr[pr >= 0]
    assert sorted(rows.tolist()) == list(range(off[-1]))  # bijection onto [0, P_in)
    for p in range(T * K):
        assert (pr[p] >= 0) == bool(mask.ravel()[p])
        if pr[p] >= 0:
            assert sp[pr[p]] == p
    x = rng.standard_normal((T, 5))
    xp = oracle.permute_rows(x, sp, K)
    for r, p in enumerate(sp):
        assert (xp[r] == x[p // K]).all()


# ---------------------------------------------------------------- MLP / forward
def test_a2a_dispatch_golden_vectors():
    for c in load_golden("a2a_dispatch.json")["cases"]:
        counts, send_token, token_pos = oracle.a2a_dispatch_indices(
            np.array(c["ids"]), c["E_global"], c["ep_size"], c["cap"])
        assert counts.tolist() == c["counts"], c["name"]
        assert send_token.tolist() == c["send_token"], c["name"]
        assert token_pos.tolist() == c["token_pos"], c["name"]


def _a2a_bruteforce(ids, E_global, ep_size, cap):
    """Scalar loops: for each rank, walk the tokens in order and append a token
    the first time one of its experts belongs to that rank."""
    T, K = len(ids), len(ids[0])
    E_local = E_global // ep_size
    counts = [0] * ep_size
    send_token = [-1] * (ep_size * cap)
    token_pos = [[-1] * ep_size for _ in range(T)]
    for r in range(ep_size):
        for t in range(T):
            mine = False
            for k in range(K):
                e = int(ids[t][k])
                if 0 <= e < E_global and r * E_local <= e < (r + 1) * E_local:
                    mine = True
            if mine:
                row = r * cap + counts[r]
                send_token[row] = t
                token_pos[t][r] = row
                counts[r] += 1
    return counts, send_token, token_pos


@pytest.mark.parametrize("seed", range(5))
def test_a2a_dispatch_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    E, ep = [(8, 2), (16, 4), (12, 3), (32, 8), (6, 1)][seed]
    T, K = 37, min(4, E)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    ids[rng.random((T, K)) < 0.05] = -1  # invalid ids go nowhere
    cap = T
    got = oracle.a2a_dispatch_indices(ids, E, ep, cap)
    want = _a2a_bruteforce(ids.tolist(), E, ep, cap)
    assert got[0].tolist() == want[0]
    assert got[1].tolist() == want[1]
    assert got[2].tolist() == want[2]
    # each token reaches exactly the ranks owning its valid experts
    E_l = E // ep
    for t in range(T):
        owners = {int(e) // E_l for e in ids[t] if 0 <= e < E}
        assert {r for r in range(ep) if got[2][t, r] >= 0} == owners


@pytest.mark.parametrize("ep_size", [1, 2, 4])
def test_a2a_forward_equals_full_forward(ep_size):
    """Dispatch + per-rank local compute + gather-sum is the full layer: each
    pair is computed on exactly one rank (its expert's owner) and the ranks'
    partial sums add up; only the summation order differs."""
    rng = np.random.default_rng(7 + ep_size)
    T, H, I, E, K = 19, 16, 24, 8, 3
    x = rng.standard_normal((T, H))
    logits = rng.standard_normal((T, E))
    wgu = rng.standard_normal((E, 2 * I, H)) / 4
    wd = rng.standard_normal((E, H, I)) / 5
    ids, w = oracle.route(logits, K, True)
    full = oracle.forward(x, logits, wgu, wd, K, True)
    a2a = oracle.a2a_forward(x, ids, w, wgu, wd, E, ep_size, cap=T)
    np.testing.assert_allclose(a2a, full, rtol=1e-12, atol=1e-12)


def test_mutation_a2a_owner_rule_is_caught(monkeypatch):
    # planted mistake: experts dealt to ranks round-robin (owner e % ep_size)
    # instead of in contiguous ranges
    orig = om.a2a_dispatch_indices

    def bad_dispatch(ids, E_global, ep_size, cap):
        ids = np.asarray(ids)
        E_l = E_global // ep_size
        perm = (ids % ep_size) * E_l + ids // ep_size
        return orig(np.where(ids >= 0, perm, ids), E_global, ep_size, cap)

    monkeypatch.setattr(om, "a2a_dispatch_indices", bad_dispatch)
    monkeypatch.setattr(oracle, "a2a_dispatch_indices", bad_dispatch)
    with pytest.raises(AssertionError):
        test_a2a_dispatch_golden_vectors()


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(z), F.silu(torch.as_tensor(z)).numpy(),
                               rtol=1e-14, atol=1e-300)


def textbook_error():
    """E=1, K=1, renormalised: the layer is one dense SwiGLU MLP (torch silu and
    matmul, fp64). H == I so a transposed operand would not fail on shape."""
    rng = np.random.default_rng(11)
    T, H, I = 7, 9, 9
    x = rng.standard_normal((T, H))
    lg = rng.standard_normal((T, 1)).astype(np.float32)
    wgu = rng.standard_normal((1, 2 * I, H))
    wd = rng.standard_normal((1, H, I))
    out = oracle.forward(x, lg, wgu, wd, K=1, renormalize=True)
    xt = torch.as_tensor(x)
    ref = (F.silu(xt @ torch.as_tensor(wgu[0, :I]).T) * (xt @ torch.as_tensor(wgu[0, I:]).T)) \
        @ torch.as_tensor(wd[0]).T
    return float(np.abs(out - ref.numpy()).max())


def test_forward_textbook_dense_mlp():
    assert textbook_error() < 1e-12


def dense_error(seed, K=3, renorm=True, ep_size=1, ep_rank=0, ties=False, E=6):
    x, lg, wgu, wd = tiny_problem(seed, E=E, K=K, ties=ties)
    out = oracle.forward(x, lg, wgu, wd, K, renorm, ep_size, ep_rank)
    ref = dense_brute(x, lg, wgu, wd, K, renorm, ep_size, ep_rank)
    return float(np.abs(out - ref).max())


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("K,renorm,ep_size,ep_rank,ties", [
    (3, True, 1, 0, False), (3, False, 1, 0, True), (1, True, 1, 0, False),
    (6, True, 1, 0, True), (2, True, 2, 1, False), (4, False, 3, 0, True), (3, True, 3, 2, False)])
def test_forward_matches_dense_bruteforce(seed, K, renorm, ep_size, ep_rank, ties):
    assert dense_error(seed, K, renorm, ep_size, ep_rank, ties) < 1e-12


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("K,renorm,ep_size,ep_rank", [(3, True, 1, 0), (2, False, 1, 0),
                                                      (4, True, 2, 1), (6, True, 1, 0)])
def test_routing_on_input_matches_dense_bruteforce(seed, K, renorm, ep_size, ep_rank):
    x, lg, wgu, wd = tiny_problem(seed, K=K)
    out = oracle.forward(x, lg, wgu, wd, K, renorm, ep_size, ep_rank, routing_on_input=True)
    ref = dense_brute(x, lg, wgu, wd, K, renorm, ep_size, ep_rank, on_input=True)
    assert np.abs(out - ref).max() < 1e-12
    # SwiGLU is not linear, so the two placements of the weight differ
    other = oracle.forward(x, lg, wgu, wd, K, renorm, ep_size, ep_rank)
    assert np.abs(out - other).max() > 1e-3


def test_routing_on_input_with_unit_weight_is_output_side():
    """K = 1 with renormalisation gives every pair weight 1: MLP(1 * x) = 1 * MLP(x)."""
    x, lg, wgu, wd = tiny_problem(9, K=1)
    a = oracle.forward(x, lg, wgu, wd, 1, True, routing_on_input=True)
    b = oracle.forward(x, lg, wgu, wd, 1, True)
    np.testing.assert_array_equal(a, b)


def test_shared_output_is_added():
    x, lg, wgu, wd = tiny_problem(10)
    sh = np.random.default_rng(1).standard_normal(x.shape)
    for on_input in (False, True):
        a = oracle.forward(x, lg, wgu, wd, 3, True, routing_on_input=on_input, shared=sh)
        b = oracle.forward(x, lg, wgu, wd, 3, True, routing_on_input=on_input)
        np.testing.assert_allclose(a - b, sh, rtol=0, atol=1e-12)
    tok = np.array([4, 0, 7])
    a = oracle.forward(x, lg, wgu, wd, 3, True, tokens=tok, shared=sh)
    b = oracle.forward(x, lg, wgu, wd, 3, True, tokens=tok)
    np.testing.assert_allclose(a - b, sh[tok], rtol=0, atol=1e-12)


def test_mutation_unscaled_input_is_caught(monkeypatch):
    real = om.forward

    def bad(x, logits, wgu, wd, K, renorm, ep_size=1, ep_rank=0, tokens=None, topk=None,
            routing_on_input=False, shared=None):
        if not routing_on_input:
            return real(x, logits, wgu, wd, K, renorm, ep_size, ep_rank, tokens, topk,
                        shared=shared)
        # planted mistake: the experts see x itself, combined with unit weights
        ids, w = om.route(logits, K, renorm)
        return real(x, None, wgu, wd, K, False, ep_size, ep_rank, tokens,
                    topk=(ids, np.ones_like(w)), shared=shared)
    monkeypatch.setattr(om, "forward", bad)
    monkeypatch.setattr(oracle, "forward", bad)
    with pytest.raises(AssertionError):
        test_routing_on_input_matches_dense_bruteforce(0, 3, False, 1, 0)


def test_zero_weight_pairs_contribute_nothing():
    x, lg, wgu, wd = tiny_problem(5)
    ids, w = oracle.route(lg, 3, True)
    w = w.copy()
    w[::2, 1] = 0.0
    out = oracle.forward(x, lg, wgu, wd, 3, True, topk=(ids, w))
    ref = dense_brute(x, lg, wgu, wd, 3, True, w_override=w)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_masked_pairs_never_read():
    x, lg, wgu, wd = tiny_problem(6, E=8, K=4)
    base = oracle.forward(x, lg, wgu, wd, 4, True, ep_size=2, ep_rank=0)
    wgu2, wd2 = wgu.copy(), wd.copy()
    wgu2[4:] = np.nan
    wd2[4:] = np.nan
    out = oracle.forward(x, lg, wgu2, wd2, 4, True, ep_size=2, ep_rank=0)
    assert np.array_equal(out, base)  # bit-identical, and finite
    # scrambling which non-local expert a masked pair names changes nothing
    ids, w = oracle.route(lg, 4, True)
    ids2 = ids.copy()
    nl = ids2 >= 4
    ids2[nl] = 4 + (ids2[nl] - 4 + 1) % 4
    out2 = oracle.forward(x, lg, wgu, wd, 4, True, ep_size=2, ep_rank=0, topk=(ids2, w))
    assert np.array_equal(out2, base)


def test_ep_partial_outputs_sum_to_full():
    x, lg, wgu, wd = tiny_problem(8, E=12, K=4)
    full = oracle.forward(x, lg, wgu, wd, 4, True)
    parts = sum(oracle.forward(x, lg, wgu, wd, 4, True, ep_size=4, ep_rank=r) for r in range(4))
    np.testing.assert_allclose(parts, full, atol=1e-12)


def staged_forward(x, lg, wgu, wd, K, renorm, ep_size, ep_rank, ro, rs, slot_expert):
    """Slot-indexed pipeline built from the oracle's stage functions."""
    E = wgu.shape[0]
    El = E // ep_size
    I = wd.shape[2]
    ids, w = oracle.route(lg, K, renorm)
    slot, wm, mask = oracle.slot_map(ids, w, E, ep_size, ep_rank, ro, rs)
    S = len(slot_expert)
    off, sp, pr = oracle.permute_indices(slot, mask, S)
    xp = oracle.permute_rows(x, sp, K)
    local = wgu[ep_rank * El:(ep_rank + 1) * El]
    local_d = wd[ep_rank * El:(ep_rank + 1) * El]
    sw = local[np.asarray(slot_expert)]
    sd = local_d[np.asarray(slot_expert)]
    a = oracle.grouped_gate_up(xp, off, sw, I)
    y = oracle.grouped_down(a, off, sd)
    return oracle.combine_rows(y, pr, wm, K)


@pytest.mark.parametrize("ep_size,ep_rank,reps", [(1, 0, []), (1, 0, [2, 0, 5]), (2, 1, [1]),
                                                   (3, 0, [0, 1])])
def test_stage_pipeline_with_slots_matches_dense(ep_size, ep_rank, reps):
    x, lg, wgu, wd = tiny_problem(9, T=17, E=6 if ep_size != 2 else 8, K=3)
    El = wgu.shape[0] // ep_size
    ro, rs, se = build_slot_table(El, reps)
    out = staged_forward(x, lg, wgu, wd, 3, True, ep_size, ep_rank, ro.numpy(), rs.numpy(),
                         se.numpy())
    ref = dense_brute(x, lg, wgu, wd, 3, True, ep_size, ep_rank)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    # the other replica choice ((t+1) mod r) gives the same output
    if reps:
        ro2, rs2 = ro.numpy(), rs.numpy().copy()
        for lid in range(El):
            a, b = ro2[lid], ro2[lid + 1]
            rs2[a:b] = np.roll(rs2[a:b], -1)
        out2 = staged_forward(x, lg, wgu, wd, 3, True, ep_size, ep_rank, ro2, rs2, se.numpy())
        np.testing.assert_allclose(out2, ref, atol=1e-12)


def test_generator_workload_roundtrip():
    """The generator's small workloads run through the oracle and the
    identity slot table equals expert-indexed compute."""
    cfg = WorkloadConfig("t", T=9, H=16, I=24, E=5, K=2, renormalize=True, dtype="bf16",
                         router="gauss_bias", bias_std=0.5)
    inp = make_inputs(cfg)
    inp2 = make_inputs(cfg)
    assert torch.equal(inp.x, inp2.x) and torch.equal(inp.w_down, inp2.w_down)
    assert torch.equal(inp.logits, inp2.logits)
    ro, rs = identity_slot_table(5)
    out = oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, 2, True)
    se = torch.arange(5, dtype=torch.int32)
    st = staged_forward(inp.x.float().numpy(), inp.logits.numpy(), inp.w_gate_up.float().numpy(),
                        inp.w_down.float().numpy(), 2, True, 1, 0, ro.numpy(), rs.numpy(), se.numpy())
    np.testing.assert_allclose(out, st, atol=1e-12)
    sw = slot_weights(inp.w_down, torch.tensor([4, 0], dtype=torch.int32))
    assert torch.equal(sw[0], inp.w_down[4]) and torch.equal(sw[1], inp.w_down[0])


# ---------------------------------------------------------------- planted mistakes
def test_mutation_silu_sign_is_caught(monkeypatch):
    monkeypatch.setattr(om, "silu", lambda z: z / (1.0 + np.exp(z)))
    assert textbook_error() > 1e-3


def test_mutation_gate_up_swap_is_caught(monkeypatch):
    def bad(xrows, w_gate, w_up, w_down):
        x = om._f64(xrows)
        return (om.silu(x @ om._f64(w_up).T) * (x @ om._f64(w_gate).T)) @ om._f64(w_down).T
    monkeypatch.setattr(om, "swiglu_mlp", bad)
    assert textbook_error() > 1e-3


def test_mutation_transposed_down_is_caught(monkeypatch):
    def bad(xrows, w_gate, w_up, w_down):
        x = om._f64(xrows)
        return (om.silu(x @ om._f64(w_gate).T) * (x @ om._f64(w_up).T)) @ om._f64(w_down)
    monkeypatch.setattr(om, "swiglu_mlp", bad)
    assert textbook_error() > 1e-3


def test_mutation_tie_order_is_caught(monkeypatch):
    def bad(logits, K):
        l = om._f64(logits)
        ids = np.broadcast_to(-np.arange(l.shape[1]), l.shape)
        return np.lexsort((ids, -l), axis=-1)[:, :K].astype(np.int32)
    monkeypatch.setattr(om, "topk_ids", bad)
    with pytest.raises(AssertionError):
        test_route_golden_vectors()


def test_mutation_nonlocal_remap_is_caught(monkeypatch):
    orig = om.ep_mask_and_remap

    def bad(ids, w, start, E_local):
        lid, wm, mask = orig(ids, w, start, E_local)
        lid = lid.copy()
        lid[~mask] = 0
        return lid, wm, mask
    monkeypatch.setattr(om, "ep_mask_and_remap", bad)
    with pytest.raises(AssertionError):
        test_slot_map_golden_vectors()


def test_mutation_unstable_slot_order_is_caught(monkeypatch):
    orig = om.permute_indices

    def bad(slot, mask, S):
        off, sp, pr = orig(slot, mask, S)
        sp = sp.copy()
        for s in range(S):
            sp[off[s]:off[s + 1]] = sp[off[s]:off[s + 1]][::-1]
        return off, sp, pr
    monkeypatch.setattr(om, "permute_indices", bad)
    monkeypatch.setattr(oracle, "permute_indices", bad)
    with pytest.raises(AssertionError):
        test_permute_golden_vectors()


def test_mutation_unmasked_weights_are_caught(monkeypatch):
    orig = om.ep_mask_and_remap

    def bad(ids, w, start, E_local):
        lid, wm, mask = orig(ids, w, start, E_local)
        return lid, om._f64(w), np.ones_like(mask)
    monkeypatch.setattr(om, "ep_mask_and_remap", bad)
    with pytest.raises(AssertionError):
        test_slot_map_golden_vectors()


def test_mutation_renorm_after_mask_is_caught(monkeypatch):
    orig = om.ep_mask_and_remap

    def bad(ids, w, start, E_local):
        lid, wm, mask = orig(ids, w, start, E_local)
        s = wm.sum(axis=1, keepdims=True)
        return lid, np.where(s > 0, wm / np.where(s > 0, s, 1), 0), mask
    monkeypatch.setattr(om, "ep_mask_and_remap", bad)
    assert dense_error(1, 3, True, 3, 0) > 1e-3
