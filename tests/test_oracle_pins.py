"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Each test names the passage or the closed form it relies on.  Together they
are meant to catch a plausible slip anywhere in the oracle: a dropped gate, a
floor instead of a ceiling, positions counted in the wrong order or after the
capacity cut, a transposed weight, a wrong argmax tie rule, a missing bias,
a wrong normalisation of f or P.
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from golden_util import keyed, rows

ALPHA = 0.01


def _onehot_logits(assign, N, rng, scale=10.0, noise=0.1):
    T = len(assign)
    h = rng.uniform(-noise, noise, size=(T, N))
    h[np.arange(T), assign] += scale
    return h


# ---------------------------------------------------------------- capacity

def test_capacity_worked_examples():
    g = keyed("lp_capacity_512_8.txt")
    assert g["T"] / g["N"] == g["even_share"]
    assert oracle.capacity(g["T"], g["N"], g["c"]) == g["capacity"]          # 96
    k = keyed("kb_capacity_16_4.txt")
    assert oracle.capacity(k["T"], k["N"], k["c"]) == k["capacity"]          # 4
    b = keyed("bh_hand_example.txt")
    # five tokens over three experts: capacity 2 needs rounding up (a floor gives 1)
    assert oracle.capacity(b["tokens"], b["experts"], 1.0) == b["capacity"]
    # the five workload shapes
    for (T, N, c), C in {(64, 4, 1.25): 20, (4096, 8, 1.25): 640, (16384, 128, 1.0): 128,
                         (32768, 128, 1.25): 320, (131072, 2048, 1.0): 64}.items():
        assert oracle.capacity(T, N, c) == C
    assert oracle.capacity(100, 4, 0.0) == 0
    assert oracle.capacity(100, 4, 1.0, capacity_override=7) == 7


# ---------------------------------------------------------------- routing

def test_softmax_table_argmax_and_derived_loss():
    """[MS] "Expert Capacity": printed softmax rows and the expert each token goes to."""
    tab = np.array([[float(v) for v in r] for r in rows("ms_softmax_table.txt")])
    p, sel = tab[:, :4], tab[:, 4].astype(np.int32)
    h = np.log(np.where(p > 0, p, 1e-12))
    r = oracle.route(h, c=1.0, alpha=ALPHA)
    assert np.array_equal(r["expert_idx"], sel)
    # derived here: loads, mean probabilities, the loss, and which tokens overflow at c=1
    assert list(r["load"]) == [4, 0, 1, 0]
    assert np.allclose(r["P"], [0.54, 0.12, 0.20, 0.14], atol=1e-9)
    assert r["aux"] == pytest.approx(ALPHA * 4 * 0.472, rel=1e-9)
    assert r["C"] == 2
    assert list(r["drop"]) == [0, 0, 1, 1, 0]
    assert list(r["position"]) == [0, 1, 2, 3, 0]
    np.testing.assert_allclose(r["gate"], p[np.arange(5), sel], rtol=1e-9)


def test_fp_examples_balanced_and_skewed():
    """[MS] "Differentiable Load Balancing Loss": sum f.P = 0.25 balanced, 0.34 skewed."""
    ex = {}
    for r in rows("ms_fp_examples.txt"):
        vals = [float(v) for v in r[1:] if v != "|"]
        ex[r[0]] = (np.array(vals[0:4]), np.array(vals[4:8]), vals[8])
    # balanced: four tokens whose probability vectors are rotations of one vector
    base = np.array([0.4, 0.3, 0.2, 0.1])
    h = np.log(np.stack([np.roll(base, t) for t in range(4)]))
    r = oracle.route(h, c=1.0, alpha=ALPHA)
    f, P, s = ex["balanced"]
    np.testing.assert_allclose(r["load"] / 4.0, f)
    np.testing.assert_allclose(r["P"], P, atol=1e-12)
    assert r["aux"] == pytest.approx(ALPHA * 4 * s, rel=1e-12)
    # skewed: 7 tokens with p = (0.4857.., 0.1714.. x3), 3 with 0.5 on experts 1, 2, 3
    rows7 = np.tile([3.4 / 7, 1.2 / 7, 1.2 / 7, 1.2 / 7], (7, 1))
    rows3 = np.array([[0.2, 0.5, 0.15, 0.15], [0.2, 0.15, 0.5, 0.15], [0.2, 0.15, 0.15, 0.5]])
    h = np.log(np.vstack([rows7, rows3]))
    r = oracle.route(h, c=1.0, alpha=ALPHA)
    f, P, s = ex["skewed"]
    np.testing.assert_allclose(r["load"] / 10.0, f)
    np.testing.assert_allclose(r["P"], P, atol=1e-12)
    assert r["aux"] == pytest.approx(ALPHA * 4 * s, rel=1e-12)        # 1.36 alpha


def test_sixteen_tokens_four_experts():
    """[KB] "16 token、4 Expertで考える": loads [7,4,3,2], C=4, 3 overflow from E1."""
    g = keyed("kb_capacity_16_4.txt")
    rng = np.random.default_rng(5)
    assign = np.repeat(np.arange(4), g["loads"])
    for trial in range(5):
        perm = rng.permutation(assign)
        r = oracle.route(_onehot_logits(perm, 4, rng), c=g["c"], alpha=ALPHA)
        assert r["C"] == g["capacity"]
        assert list(r["load"]) == g["loads"]
        dropped = np.flatnonzero(r["drop"])
        assert len(dropped) == g["overflow_count"]
        assert set(perm[dropped]) == {g["overflow_expert"]}
        # the overflow tokens are that expert's 5th..7th tokens in token order
        e0 = np.flatnonzero(perm == 0)
        assert list(dropped) == list(e0[4:7])


def test_hand_example_overflow_passes_through():
    """[BH] steps 5-13 with the errata: Z5 = [5,3,1] scores [2,3,4] -> C, C is full,
    Z5 leaves the layer unchanged.  Switch rows A and B and Z1..Z4 are constructed here
    (the page prints them only as images); row C is the page's."""
    g = keyed("bh_hand_example.txt")
    W_r = np.array([[0, 0, 2], [0, 1, 0], g["switch_row_C"]], dtype=np.float32)
    Z = np.array([[0, 0, 3], [0, 2, 1], [0, 3, -1], [0, 3, 1], g["Z5"]], dtype=np.float32)
    h = oracle.logits(Z, W_r)
    np.testing.assert_array_equal(h[4], g["Z5_scores"])
    rng = np.random.default_rng(0)
    W_in = rng.normal(0, 0.5, size=(3, 4, 3)).astype(np.float32)
    W_out = rng.normal(0, 0.5, size=(3, 3, 4)).astype(np.float32)
    r = oracle.forward(Z, W_r, None, W_in, W_out, c=1.0, alpha=ALPHA)
    assert r["C"] == g["capacity"]
    assert r["expert_idx"][0] == g["Z1_expert"]
    assert r["expert_idx"][4] == g["Z5_expert"]
    assert list(r["expert_idx"]) == [0, 2, 1, 2, 2]
    assert r["position"][4] == 2 and r["drop"][4] == 1
    assert np.array_equal(r["out"][4], Z[4].astype(np.float64))       # passed through
    # kept tokens: x + p * relu(x W_in^T) W_out^T, evaluated with library matmuls
    for t in range(4):
        e = r["expert_idx"][t]
        p = softmax(h[t])[e]
        E = np.maximum(Z[t].astype(np.float64) @ W_in[e].T.astype(np.float64), 0) @ W_out[e].T.astype(np.float64)
        np.testing.assert_allclose(r["out"][t], Z[t] + p * E, rtol=1e-12, atol=1e-12)
        assert not np.allclose(E, 0)


# ---------------------------------------------------------------- closed forms

def test_aux_equals_alpha_when_f_uniform():
    """[LP 3.3] aux = alpha at uniform routing; holds for any P when f is uniform."""
    rng = np.random.default_rng(1)
    N, T = 8, 64
    h = rng.normal(0, 1, size=(T, N))
    h[np.arange(T), np.arange(T) % N] += 20.0
    r = oracle.route(h, c=2.0, alpha=ALPHA)
    assert np.all(r["load"] == T // N)
    assert r["aux"] == pytest.approx(ALPHA, rel=1e-12)


def test_aux_equals_alpha_when_p_uniform_and_ties_go_low():
    """All-equal logits: P uniform -> aux = alpha; exact ties pick the lowest index."""
    T, N = 10, 5
    r = oracle.route(np.full((T, N), 0.3), c=1.0, alpha=ALPHA)
    assert np.all(r["expert_idx"] == 0)
    np.testing.assert_allclose(r["gate"], 1.0 / N, rtol=1e-15)
    assert r["aux"] == pytest.approx(ALPHA, rel=1e-12)
    h = np.array([[0.0, 1.0, 3.0, 3.0, -2.0]])
    assert oracle.route(h, c=1.0)["expert_idx"][0] == 2


def test_alpha_is_not_a_lower_bound():
    """Two pages call alpha the minimum; it is not in general.  Counterexample
    N=2, T=3: aux = 0.8956 alpha (the reading: only 'alpha under uniform f or P')."""
    p = np.array([[0.51, 0.49], [0.51, 0.49], [0.01, 0.99]])
    r = oracle.route(np.log(p), c=2.0, alpha=ALPHA)
    f = np.array([2 / 3, 1 / 3])
    P = p.mean(axis=0)
    assert r["aux"] == pytest.approx(ALPHA * 2 * (f @ P), rel=1e-12)
    assert r["aux"] < ALPHA


def test_single_expert_gate_one():
    rng = np.random.default_rng(2)
    r = oracle.route(rng.normal(size=(17, 1)), c=1.0, alpha=ALPHA)
    assert np.all(r["gate"] == 1.0)
    assert r["aux"] == ALPHA
    assert np.array_equal(r["position"], np.arange(17))


def test_router_bias_only():
    """W_r = 0: every token goes to argmax b; positions 0..T-1; drops max(T-C, 0)."""
    rng = np.random.default_rng(3)
    T, d, N, c = 40, 16, 6, 1.5
    b = rng.normal(size=N).astype(np.float32)
    x = rng.normal(size=(T, d)).astype(np.float32)
    r = oracle.route(oracle.logits(x, np.zeros((N, d), np.float32), b), c=c, alpha=ALPHA)
    istar = int(np.argmax(b))
    C = int(np.ceil(c * T / N))
    assert np.all(r["expert_idx"] == istar)
    assert np.array_equal(r["position"], np.arange(T))
    assert int(r["drop"].sum()) == max(T - C, 0)
    sm = softmax(b.astype(np.float64))
    np.testing.assert_allclose(r["gate"], sm[istar], rtol=1e-12)
    assert r["aux"] == pytest.approx(ALPHA * N * sm[istar], rel=1e-12)


def test_capacity_zero_drops_everything():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(9, 8)).astype(np.float32)
    W_r = rng.normal(size=(3, 8)).astype(np.float32)
    W_in = rng.normal(size=(3, 16, 8)).astype(np.float32)
    W_out = rng.normal(size=(3, 8, 16)).astype(np.float32)
    r = oracle.forward(x, W_r, None, W_in, W_out, c=0.0)
    assert r["C"] == 0 and np.all(r["drop"] == 1)
    assert np.array_equal(r["out"], x.astype(np.float64))


# ---------------------------------------------------------------- library routines

def test_logits_match_library_matmul():
    rng = np.random.default_rng(6)
    T, d, N = 37, 29, 11
    x = rng.normal(size=(T, d)).astype(np.float32)
    W_r = rng.normal(size=(N, d)).astype(np.float32)
    b = rng.normal(size=N).astype(np.float32)
    ref = x.astype(np.float64) @ W_r.T.astype(np.float64) + b
    np.testing.assert_allclose(oracle.logits(x, W_r, b), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.logits(x, W_r), ref - b, rtol=1e-12, atol=1e-12)


def test_dense_special_case_is_two_matmul_mlp():
    """N = 1 and capacity >= T: out = x + relu(x W_in^T) W_out^T exactly (gate = 1)."""
    rng = np.random.default_rng(7)
    T, d, F = 23, 12, 20
    x = rng.normal(size=(T, d)).astype(np.float32)
    W_r = rng.normal(size=(1, d)).astype(np.float32)
    W_in = rng.normal(size=(1, F, d)).astype(np.float32)
    W_out = rng.normal(size=(1, d, F)).astype(np.float32)
    r = oracle.forward(x, W_r, None, W_in, W_out, c=1.0)
    x64 = x.astype(np.float64)
    E = np.maximum(x64 @ W_in[0].T.astype(np.float64), 0) @ W_out[0].T.astype(np.float64)
    assert not np.any(r["drop"])
    np.testing.assert_allclose(r["out"], x64 + E, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["E"], E, rtol=1e-12, atol=1e-12)


def test_token_output_agrees_with_combine():
    rng = np.random.default_rng(8)
    T, d, F, N = 15, 8, 24, 3
    x = rng.normal(size=(T, d)).astype(np.float32)
    W_r = rng.normal(size=(N, d)).astype(np.float32)
    W_in = rng.normal(size=(N, F, d)).astype(np.float32)
    W_out = rng.normal(size=(N, d, F)).astype(np.float32)
    r = oracle.forward(x, W_r, None, W_in, W_out, c=1.0)
    for t in range(T):
        e = r["expert_idx"][t]
        o, E = oracle.token_output(x[t], r["drop"][t], r["gate"][t], W_in[e], W_out[e])
        assert np.array_equal(o, r["out"][t])
        assert np.array_equal(E, r["E"][t])


# ---------------------------------------------------------------- brute force / invariants

@pytest.mark.parametrize("T,N,c", [(5, 3, 1.0), (6, 2, 1.0), (4, 3, 0.5), (6, 3, 2.0)])
def test_brute_force_all_assignments(T, N, c):
    """Every one of the N^T assignments: positions against the quadratic rule
    (count earlier tokens of the same expert), drops against sum max(load - C, 0),
    aux against a direct evaluation with scipy's softmax."""
    rng = np.random.default_rng(T * 10 + N)
    C = int(np.ceil(c * T / N))
    for assign in itertools.product(range(N), repeat=T):
        assign = np.array(assign)
        h = _onehot_logits(assign, N, rng)
        r = oracle.route(h, c=c, alpha=ALPHA)
        assert np.array_equal(r["expert_idx"], assign)
        pos = np.array([np.sum(assign[:t] == assign[t]) for t in range(T)])
        assert np.array_equal(r["position"], pos)
        load = np.bincount(assign, minlength=N)
        assert int(r["drop"].sum()) == int(np.maximum(load - C, 0).sum())
        assert np.array_equal(r["drop"], (pos >= C).astype(np.uint8))
        p = softmax(h, axis=1)
        assert r["aux"] == pytest.approx(ALPHA * N * np.sum(load / T * p.mean(axis=0)), rel=1e-12)


def test_routing_invariants_random():
    rng = np.random.default_rng(9)
    T, N, c = 2000, 16, 1.0
    h = rng.normal(size=(T, N)) + rng.normal(size=N) * 0.5
    r = oracle.route(h, c=c, alpha=ALPHA)
    assert r["load"].sum() == T
    assert abs(r["P"].sum() - 1.0) <= 1e-12
    for e in range(N):
        toks = np.flatnonzero(r["expert_idx"] == e)
        assert np.array_equal(r["position"][toks], np.arange(len(toks)))
    kept = int((r["drop"] == 0).sum())
    assert kept == int(np.minimum(r["load"], r["C"]).sum())


def test_relabelling_experts_permutes_routing_only():
    rng = np.random.default_rng(10)
    T, d, F, N = 50, 16, 32, 5
    x = rng.normal(size=(T, d)).astype(np.float32)
    W_r = rng.normal(size=(N, d)).astype(np.float32)
    W_in = rng.normal(size=(N, F, d)).astype(np.float32)
    W_out = rng.normal(size=(N, d, F)).astype(np.float32)
    perm = rng.permutation(N)              # new expert j is old expert perm[j]
    a = oracle.forward(x, W_r, None, W_in, W_out, c=1.0)
    b = oracle.forward(x, W_r[perm], None, W_in[perm], W_out[perm], c=1.0)
    inv = np.argsort(perm)
    assert np.array_equal(b["expert_idx"], inv[a["expert_idx"]])
    assert np.array_equal(a["position"], b["position"])
    np.testing.assert_allclose(a["gate"], b["gate"], rtol=1e-14)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-13, atol=1e-13)
    assert a["aux"] == pytest.approx(b["aux"], rel=1e-13)


# ---------------------------------------------------------------- top-k routing (next row)

def test_topk_hospital_example():
    """llm-papers-study 3.1: top-2 picks the two best experts, weighted by their
    softmax probabilities (0.6 and 0.3); top-1 picks the best alone."""
    g = keyed("lp_hospital_top2.txt")
    p = np.array(g["p"], dtype=np.float64)
    h = np.log(p)[None, :]
    r2 = oracle.route_topk(h, 2, c=10.0)
    assert list(r2["expert_idx"][0]) == [int(v) for v in g["top2_experts"]]
    assert np.allclose(r2["gate"][0], g["top2_weights"], rtol=0, atol=1e-12)
    r1 = oracle.route_topk(h, 1, c=10.0)
    assert r1["expert_idx"][0, 0] == int(g["top1_expert"])
    # output = x + 0.6 E_0(x) + 0.3 E_1(x), with the experts evaluated by a library matmul
    rng = np.random.default_rng(7)
    d, F, N = 4, 6, 3
    x = rng.standard_normal((1, d)).astype(np.float32)
    W_in = rng.standard_normal((N, F, d)).astype(np.float32)
    W_out = rng.standard_normal((N, d, F)).astype(np.float32)
    out, E = oracle.combine_topk(x, r2["expert_idx"], r2["gate"], r2["drop"], W_in, W_out)
    ex = [np.maximum(W_in[e].astype(np.float64) @ x[0], 0) @ W_out[e].T.astype(np.float64)
          for e in range(N)]
    want = x[0] + 0.6 * ex[0] + 0.3 * ex[1]
    assert np.allclose(out[0], want, rtol=1e-12, atol=1e-12)
    assert np.allclose(E[0, 0], ex[0]) and np.allclose(E[0, 1], ex[1])


def test_topk_capacity_doubles_for_two_choices():
    """llm-papers-study 3.2 point (2): one expert per token at least halves the
    capacity; read as: k choices take k times the top-1 capacity.  With section
    3.4's 512 tokens / 8 experts / factor 1.5 (capacity 96), top-2 gives 192."""
    g = keyed("lp_capacity_512_8.txt")
    assert oracle.capacity_topk(g["T"], g["N"], 1, g["c"]) == g["capacity"]
    assert oracle.capacity_topk(g["T"], g["N"], 2, g["c"]) == 2 * g["capacity"]


def test_topk_two_of_two_experts():
    """Closed form, N = 2 and k = 2: every token uses both experts, the gates sum
    to 1 and each expert's assignments arrive one per token, so the position of
    token t is t in both choices; capacity ceil(2 c T / 2) cuts the tail."""
    rng = np.random.default_rng(11)
    T = 37
    h = rng.standard_normal((T, 2))
    r = oracle.route_topk(h, 2, c=0.75)
    assert r["C"] == int(np.ceil(0.75 * T))
    assert np.all(np.sort(r["expert_idx"], axis=1) == [0, 1])
    assert np.allclose(r["gate"].sum(axis=1), 1.0, atol=1e-15)
    assert np.all(r["gate"][:, 0] >= r["gate"][:, 1])
    assert np.array_equal(r["position"], np.repeat(np.arange(T)[:, None], 2, axis=1))
    assert np.array_equal(r["drop"], (r["position"] >= r["C"]).astype(np.uint8))
    assert np.array_equal(r["load"], [T, T])


def test_topk_all_experts_identical_is_dense_mlp():
    """k = N with identical experts and no drops: the gates are all of softmax and
    sum to 1, so the layer is x + FFN(x), a dense two-matmul MLP (library matmul)."""
    rng = np.random.default_rng(12)
    T, d, F, N = 20, 8, 12, 3
    x = rng.standard_normal((T, d)).astype(np.float32)
    w1 = rng.standard_normal((F, d)).astype(np.float32)
    w2 = rng.standard_normal((d, F)).astype(np.float32)
    W_in = np.repeat(w1[None], N, axis=0)
    W_out = np.repeat(w2[None], N, axis=0)
    h = rng.standard_normal((T, N))
    r = oracle.route_topk(h, N, c=2.0)
    assert not r["drop"].any()
    out, _ = oracle.combine_topk(x, r["expert_idx"], r["gate"], r["drop"], W_in, W_out)
    dense = x.astype(np.float64) + np.maximum(x.astype(np.float64) @ w1.T.astype(np.float64), 0) \
        @ w2.T.astype(np.float64)
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-11)


def test_topk_uniform_load_gives_alpha():
    """The loss keeps aux = alpha when f is uniform: token t prefers expert t mod N
    then t + 1 mod N, so every expert receives the same number of assignments."""
    rng = np.random.default_rng(13)
    N, T = 4, 40
    h = rng.uniform(-0.1, 0.1, size=(T, N))
    h[np.arange(T), np.arange(T) % N] += 10.0
    h[np.arange(T), (np.arange(T) + 1) % N] += 5.0
    r = oracle.route_topk(h, 2, c=1.0)
    assert np.all(r["load"] == 2 * T // N)
    assert r["aux"] == pytest.approx(ALPHA, rel=1e-12)


def test_topk_ties_go_low_and_k1_is_top1():
    """Equal logits: the choices are experts 0, 1, ... in order; with k = 1 the
    top-k routing is the top-1 routing."""
    r = oracle.route_topk(np.zeros((3, 5)), 3, c=5.0)
    assert np.array_equal(r["expert_idx"], [[0, 1, 2]] * 3)
    assert np.allclose(r["gate"], 0.2)
    rng = np.random.default_rng(14)
    h = rng.standard_normal((300, 7))
    a = oracle.route(h, 1.1)
    b = oracle.route_topk(h, 1, 1.1)
    for k in ("expert_idx", "position", "drop"):
        assert np.array_equal(a[k], b[k][:, 0]), k
    assert np.array_equal(a["gate"], b["gate"][:, 0])
    assert np.array_equal(a["load"], b["load"])
    assert a["aux"] == b["aux"]


@pytest.mark.parametrize("T,N,c", [(4, 3, 0.5), (5, 3, 0.8), (4, 4, 0.5)])
def test_topk_brute_force_positions(T, N, c):
    """Every ordering of N experts per token (tiny T): positions by the quadratic
    rule over the (token, choice) order, drops by the capacity, loads by count."""
    rng = np.random.default_rng(15)
    perms = list(itertools.permutations(range(N)))
    for combo in itertools.product(range(len(perms)), repeat=T):
        if rng.random() > 0.2:
            continue
        h = np.zeros((T, N))
        for t, pi in enumerate(combo):
            h[t, list(perms[pi])] = [10.0 - q for q in range(N)]  # rank order = the permutation
        r = oracle.route_topk(h, 2, c)
        seq = [perms[pi][j] for pi in combo for j in range(2)]
        assert np.array_equal(r["expert_idx"].ravel(), seq)
        C = int(np.ceil(2 * c * T / N))
        for a, e in enumerate(seq):
            pos = sum(1 for b in range(a) if seq[b] == e)
            assert r["position"].ravel()[a] == pos
            assert r["drop"].ravel()[a] == (pos >= C)
        assert np.array_equal(r["load"], np.bincount(seq, minlength=N))
