"""Pins for the fp64 oracle: checks against facts fixed by the pages and by
mathematics, never against the oracle itself.

The rule being pinned is the Gated DeltaNet state update and the tree
verification it implies (Trees from Marginals technical summary, Methodology,
"3. Rollback-Free Tree Verification for GDN"):  S_t = a_t S_{t-1}(I - b_t k_t k_t^T)
+ b_t v_t k_t^T, o_t = S_t q_t, run from S0 along each node's root-to-node path
of a topologically sorted tree, and the delayed commit of the accepted node's
state.

Each test names the kind of pin: a hand-worked example (golden fixture),
a closed form for a special case, an independently written recurrence
(different orientation), brute force over the branches of tiny trees, or an
invariant that must hold exactly.
"""
import itertools

import numpy as np
import pytest

import oracle
from gdn_inputs import tree_best_first, tree_chain, tree_uniform, rng_for
from tests.conftest import read_golden


# ----------------------------------------------------------------------------
# helpers written for the tests (independent of oracle/gdn_oracle.c)
# ----------------------------------------------------------------------------

def rand_case(seed, B, N, Hk, Hv, dk, dv, tree="uniform", unit_qk=True):
    rng = np.random.default_rng(seed)
    if tree == "uniform":
        parent = tree_uniform(rng, B, N)
    elif tree == "chain":
        parent = tree_chain(B, N)
    else:
        parent = tree_best_first(rng, B, N, max_depth=4)
    q = rng.standard_normal((B, N, Hk, dk))
    k = rng.standard_normal((B, N, Hk, dk))
    if unit_qk:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, N, Hv, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((B, N, Hv)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, N, Hv))))
    S0 = 0.3 * rng.standard_normal((B, Hv, dv, dk))
    return dict(q=q, k=k, v=v, g=g, beta=beta, parent=parent, S0=S0)


def paths(parent_row):
    """root..i path of every node, by following parent links."""
    out = []
    for i in range(len(parent_row)):
        p, s = [], i
        while s >= 0:
            p.append(s)
            s = parent_row[s]
        out.append(p[::-1])
    return out


def children_lists(parent_row):
    ch = [[] for _ in parent_row]
    for i, p in enumerate(parent_row):
        if p >= 0:
            ch[p].append(i)
    return ch


def kv_head(h, Hk, Hv):
    return h // (Hv // Hk)


def chain_recurrence_dkdv(q, k, v, g, beta, S0_dvdk):
    """Token-by-token GDN recurrence written in the other orientation (state
    M of shape d_k x d_v, M_t = a_t (I - b_t k_t k_t^T) M_{t-1} + b_t k_t v_t^T,
    o_t = M_t^T q_t).  Returns the outputs and the final state as d_v x d_k."""
    M = S0_dvdk.T.copy()
    dk = M.shape[0]
    outs = []
    for t in range(len(k)):
        a = np.exp(g[t])
        kt = k[t][:, None]
        M = a * (np.eye(dk) - beta[t] * kt @ kt.T) @ M + beta[t] * kt @ v[t][None, :]
        outs.append(M.T @ q[t])
    return np.array(outs), M.T


def verify(case, **kw):
    return oracle.verify(case["q"], case["k"], case["v"], case["g"], case["beta"],
                         case["parent"], case["S0"], **kw)


def commit(case, accepted, **kw):
    return oracle.commit(case["k"], case["v"], case["g"], case["beta"], case["parent"],
                         case["S0"], accepted, **kw)


# ----------------------------------------------------------------------------
# (vi) hand-worked dyadic example (golden fixture)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("which", ["tree", "chain"])
@pytest.mark.parametrize("d", [1, 64])
def test_dyadic_worked_example(which, d):
    gold = read_golden("dyadic_tree3.txt")
    parent = np.array([gold["parent_" + which]], dtype=np.int32)
    N = parent.shape[1]
    e0 = np.zeros(d)
    e0[0] = 1.0
    q = np.tile(e0, (1, N, 1, 1))
    k = q.copy()
    v = np.zeros((1, N, 1, d))
    v[0, :, 0, 0] = gold["v"]
    g = np.full((1, N, 1), gold["g"][0])
    beta = np.full((1, N, 1), gold["beta"][0])
    S0 = np.zeros((1, 1, d, d))
    S0[0, 0, 0, 0] = gold["S0"][0]
    o = oracle.verify(q, k, v, g, beta, parent, S0)
    assert np.array_equal(o[0, :, 0, 0], np.array(gold["o_" + which]))
    assert not np.any(o[0, :, 0, 1:])
    for a in range(N):
        Sn = oracle.commit(k, v, g, beta, parent, S0, np.array([a], np.int32))
        assert Sn[0, 0, 0, 0] == gold["commit_" + which][a]
        assert np.count_nonzero(Sn) <= 1


# ----------------------------------------------------------------------------
# (i) b = 0: o_i = exp(G_i) S0 q_i, commit = exp(G_a) S0
# ----------------------------------------------------------------------------

def test_beta_zero_is_pure_decay():
    case = rand_case(1, B=2, N=9, Hk=2, Hv=4, dk=5, dv=3)
    case["beta"][:] = 0.0
    o = verify(case)
    B, N, Hv = case["g"].shape
    Hk = case["q"].shape[2]
    for b in range(B):
        P = paths(case["parent"][b])
        for i in range(N):
            for h in range(Hv):
                G = sum(case["g"][b, s, h] for s in P[i])
                want = np.exp(G) * case["S0"][b, h] @ case["q"][b, i, kv_head(h, Hk, Hv)]
                np.testing.assert_allclose(o[b, i, h], want, rtol=1e-13, atol=1e-15)
    acc = np.array([N - 1, 3], np.int32)
    Sn = commit(case, acc)
    for b in range(B):
        P = paths(case["parent"][b])
        for h in range(Hv):
            G = sum(case["g"][b, s, h] for s in P[acc[b]])
            np.testing.assert_allclose(Sn[b, h], np.exp(G) * case["S0"][b, h], rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------
# (ii) g = b = 0: o_i = S0 q_i  (also fixes the orientation of S0: a
# transposed state would give S0^T q)
# ----------------------------------------------------------------------------

def test_no_decay_no_write_reads_prefix_state():
    case = rand_case(2, B=1, N=6, Hk=1, Hv=2, dk=4, dv=7)
    case["beta"][:] = 0.0
    case["g"][:] = 0.0
    o = verify(case)
    for i in range(6):
        for h in range(2):
            np.testing.assert_allclose(o[0, i, h], case["S0"][0, h] @ case["q"][0, i, 0], rtol=1e-14)


# ----------------------------------------------------------------------------
# (iii) g = 0, b = 1, q_i = k_i with |k_i| = 1: S_i k_i = v_i exactly, so
# o_i = v_i for any tree and any S0 (the delta rule overwrites the slot)
# ----------------------------------------------------------------------------

def test_delta_rule_overwrite():
    case = rand_case(3, B=2, N=11, Hk=2, Hv=2, dk=6, dv=5)
    case["g"][:] = 0.0
    case["beta"][:] = 1.0
    case["q"] = case["k"].copy()
    o = verify(case)
    np.testing.assert_allclose(o, case["v"], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# (iv) a chain tree is the plain sequence: it equals a token-by-token
# recurrence written in the other orientation
# ----------------------------------------------------------------------------

def test_chain_equals_token_recurrence():
    case = rand_case(4, B=2, N=12, Hk=2, Hv=4, dk=5, dv=6, tree="chain")
    o = verify(case)
    Sn = commit(case, np.array([11, 5], np.int32))
    for b, h in itertools.product(range(2), range(4)):
        kh = kv_head(h, 2, 4)
        outs, Sfin = chain_recurrence_dkdv(case["q"][b, :, kh], case["k"][b, :, kh], case["v"][b, :, h],
                                           case["g"][b, :, h], case["beta"][b, :, h], case["S0"][b, h])
        np.testing.assert_allclose(o[b, :, h], outs, rtol=1e-11, atol=1e-13)
        if b == 0:
            np.testing.assert_allclose(Sn[b, h], Sfin, rtol=1e-11, atol=1e-13)
        else:
            _, S6 = chain_recurrence_dkdv(case["q"][b, :6, kh], case["k"][b, :6, kh], case["v"][b, :6, h],
                                          case["g"][b, :6, h], case["beta"][b, :6, h], case["S0"][b, h])
            np.testing.assert_allclose(Sn[b, h], S6, rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------------------
# (v) brute force over branches: every root-to-leaf branch is run as a plain
# sequence; each node must get the same output from every branch through it,
# and that output must equal the oracle's
# ----------------------------------------------------------------------------

def brute_force_tree(case):
    B, N, Hk, dk = case["q"].shape
    Hv, dv = case["v"].shape[2:]
    out = np.full((B, N, Hv, dv), np.nan)
    for b in range(B):
        par = case["parent"][b]
        ch = children_lists(par)
        P = paths(par)
        leaves = [i for i in range(N) if not ch[i]]
        for leaf in leaves:
            br = P[leaf]
            for h in range(Hv):
                kh = kv_head(h, Hk, Hv)
                outs, _ = chain_recurrence_dkdv(case["q"][b, br, kh], case["k"][b, br, kh],
                                                case["v"][b, br, h], case["g"][b, br, h],
                                                case["beta"][b, br, h], case["S0"][b, h])
                for pos, node in enumerate(br):
                    if np.isnan(out[b, node, h, 0]):
                        out[b, node, h] = outs[pos]
                    else:  # a node shared by several branches: same result
                        np.testing.assert_allclose(out[b, node, h], outs[pos], rtol=1e-13, atol=1e-15)
    assert not np.isnan(out).any()
    return out


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_over_branches(seed):
    tree = ["uniform", "best_first", "chain"][seed % 3]
    case = rand_case(10 + seed, B=2, N=10, Hk=1, Hv=2, dk=4, dv=3, tree=tree)
    np.testing.assert_allclose(verify(case), brute_force_tree(case), rtol=1e-11, atol=1e-13)


def test_brute_force_forest():
    """several nodes hanging off the prefix state (a forest) is the same math"""
    case = rand_case(20, B=1, N=9, Hk=1, Hv=1, dk=3, dv=3)
    case["parent"][0] = [-1, 0, -1, 2, 0, -1, 3, 5, 1]
    np.testing.assert_allclose(verify(case), brute_force_tree(case), rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------------------
# (vii) linearity: o and S_new are linear in (S0, V) jointly
# ----------------------------------------------------------------------------

def test_linear_in_state_and_values():
    c1 = rand_case(30, B=1, N=8, Hk=1, Hv=2, dk=4, dv=5)
    c2 = dict(c1)
    rng = np.random.default_rng(31)
    c2["S0"] = rng.standard_normal(c1["S0"].shape)
    c2["v"] = rng.standard_normal(c1["v"].shape)
    a, b = 0.7, -1.3
    c3 = dict(c1)
    c3["S0"] = a * c1["S0"] + b * c2["S0"]
    c3["v"] = a * c1["v"] + b * c2["v"]
    np.testing.assert_allclose(verify(c3), a * verify(c1) + b * verify(c2), rtol=1e-11, atol=1e-12)
    acc = np.array([6], np.int32)
    np.testing.assert_allclose(commit(c3, acc), a * commit(c1, acc) + b * commit(c2, acc),
                               rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------
# (viii) subtree locality: perturbing node j's inputs changes exactly the
# outputs of j's descendants (j included); bit-exact elsewhere
# ----------------------------------------------------------------------------

def test_subtree_locality():
    case = rand_case(40, B=1, N=12, Hk=1, Hv=1, dk=4, dv=4)
    o = verify(case)
    P = paths(case["parent"][0])
    for j in range(12):
        pert = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in case.items()}
        pert["k"][0, j] += 0.25
        pert["v"][0, j] -= 0.5
        pert["g"][0, j] -= 0.1
        pert["beta"][0, j] *= 0.5
        pert["q"][0, j] += 0.3
        o2 = verify(pert)
        for i in range(12):
            if j in P[i]:
                assert not np.array_equal(o[0, i], o2[0, i])
            else:
                assert np.array_equal(o[0, i], o2[0, i])
        for a in range(12):
            same = np.array_equal(commit(case, np.array([a], np.int32)), commit(pert, np.array([a], np.int32)))
            assert same == (j not in P[a])


# ----------------------------------------------------------------------------
# (ix) relabelling: another topological order of the same tree permutes the
# outputs, bit-exactly (the oracle's arithmetic follows the paths only)
# ----------------------------------------------------------------------------

def test_relabelling_permutes_outputs():
    case = rand_case(50, B=1, N=10, Hk=1, Hv=2, dk=3, dv=4)
    par = case["parent"][0]
    rng = np.random.default_rng(51)
    # random topological order: repeatedly pick a random node whose parent is placed
    placed, order = set(), []
    while len(order) < 10:
        ready = [i for i in range(10) if i not in placed and (par[i] < 0 or par[i] in placed)]
        pick = ready[rng.integers(len(ready))]
        order.append(pick)
        placed.add(pick)
    new_of = {old: new for new, old in enumerate(order)}
    perm = np.array(order)
    c2 = {kk: vv for kk, vv in case.items()}
    for name in ("q", "k", "v", "g", "beta"):
        c2[name] = case[name][:, perm]
    c2["parent"] = np.array([[new_of[par[o]] if par[o] >= 0 else -1 for o in order]], np.int32)
    assert oracle.check_tree(c2["parent"])
    assert np.array_equal(verify(c2), verify(case)[:, perm])


# ----------------------------------------------------------------------------
# (x) the closed form (derived from the recurrence: u_i = b_i(v_i - a_i
# S_p(i) k_i), (I + X) U = diag(b)(V - diag(gamma) K S0^T),
# O = diag(gamma) Q S0^T + Y U, S_new = gamma_a S0 + sum_s D_as u_s k_s^T)
# equals the recurrence in fp64 to 1e-12
# ----------------------------------------------------------------------------

def closed_form(case, accepted=None):
    q, k, v, g, beta, parent, S0 = (case[n] for n in ("q", "k", "v", "g", "beta", "parent", "S0"))
    B, N, Hk, dk = q.shape
    Hv, dv = v.shape[2:]
    O = np.zeros((B, N, Hv, dv))
    Snew = None if accepted is None else np.zeros((B, Hv, dv, dk))
    for b in range(B):
        P = paths(parent[b])
        for h in range(Hv):
            kh = kv_head(h, Hk, Hv)
            Q, K, V = q[b, :, kh], k[b, :, kh], v[b, :, h]
            G = np.array([sum(g[b, s, h] for s in P[i]) for i in range(N)])
            gam = np.exp(G)
            X = np.zeros((N, N))
            Y = np.zeros((N, N))
            for i in range(N):
                for s in P[i]:
                    D = np.exp(G[i] - G[s])
                    if s != i:
                        X[i, s] = beta[b, i, h] * D * (K[i] @ K[s])
                    Y[i, s] = D * (Q[i] @ K[s])
            R = beta[b, :, h][:, None] * (V - gam[:, None] * (K @ S0[b, h].T))
            U = np.linalg.solve(np.eye(N) + X, R)
            O[b, :, h] = gam[:, None] * (Q @ S0[b, h].T) + Y @ U
            if accepted is not None:
                a = accepted[b]
                S = S0[b, h].copy() if a < 0 else gam[a] * S0[b, h]
                if a >= 0:
                    for s in P[a]:
                        S = S + np.exp(G[a] - G[s]) * np.outer(U[s], K[s])
                Snew[b, h] = S
    return O, Snew


@pytest.mark.parametrize("seed,tree", [(60, "uniform"), (61, "best_first"), (62, "chain")])
def test_closed_form_matches_recurrence(seed, tree):
    case = rand_case(seed, B=2, N=14, Hk=2, Hv=4, dk=6, dv=5, tree=tree)
    acc = np.array([13, -1], np.int32)
    O, Sn = closed_form(case, acc)
    o = verify(case)
    assert np.linalg.norm(o - O) <= 1e-12 * np.linalg.norm(O)
    s = commit(case, acc)
    assert np.linalg.norm(s - Sn) <= 1e-12 * np.linalg.norm(Sn)


# ----------------------------------------------------------------------------
# (xi) memoised oracle == per-path replay bit for bit; N = 1 equals one step
# done by hand
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("tree", ["uniform", "best_first", "chain"])
def test_memo_equals_replay(tree):
    case = rand_case(70, B=2, N=16, Hk=1, Hv=2, dk=5, dv=4, tree=tree)
    assert np.array_equal(verify(case, memo=True), verify(case, memo=False))
    assert np.array_equal(verify(case, memo=True, threads=1), verify(case, memo=True, threads=3))


def test_single_node_is_one_step():
    case = rand_case(71, B=1, N=1, Hk=1, Hv=1, dk=3, dv=2)
    a = np.exp(case["g"][0, 0, 0])
    bt = case["beta"][0, 0, 0]
    kk = case["k"][0, 0, 0]
    S = case["S0"][0, 0]
    S1 = a * S @ (np.eye(3) - bt * np.outer(kk, kk)) + bt * np.outer(case["v"][0, 0, 0], kk)
    np.testing.assert_allclose(verify(case)[0, 0, 0], S1 @ case["q"][0, 0, 0], rtol=1e-14)
    np.testing.assert_allclose(commit(case, np.array([0], np.int32))[0, 0], S1, rtol=1e-14)


def test_commit_minus_one_keeps_prefix_state():
    case = rand_case(72, B=2, N=5, Hk=1, Hv=1, dk=3, dv=2)
    Sn = commit(case, np.array([-1, -1], np.int32))
    assert np.array_equal(Sn, case["S0"])


def test_empty_tree():
    case = rand_case(73, B=2, N=0, Hk=1, Hv=1, dk=3, dv=2)
    assert verify(case).shape == (2, 0, 1, 2)


# ----------------------------------------------------------------------------
# ancestor sets and depth (brute force), and input validation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 7, 32, 33, 70])
def test_ancestors_brute_force(N):
    rng = np.random.default_rng(N)
    parent = np.concatenate([tree_uniform(rng, 2, N), tree_best_first(rng, 1, N, 5)])
    anc, depth = oracle.ancestors(parent)
    for b in range(parent.shape[0]):
        P = paths(parent[b])
        for i in range(N):
            bits = {s for s in range(N) if (anc[b, i, s // 32] >> (s % 32)) & 1}
            assert bits == set(P[i])
            assert depth[b, i] == len(P[i])


@pytest.mark.parametrize("bad", [[-1, 1], [-1, 0, 3], [0, 0], [-2, 0], [-1, 0, 2]])
def test_invalid_tree_rejected(bad):
    parent = np.array([bad], np.int32)
    assert not oracle.check_tree(parent)
    case = rand_case(80, B=1, N=len(bad), Hk=1, Hv=1, dk=2, dv=2)
    case["parent"] = parent
    with pytest.raises(oracle.OracleError):
        verify(case)
    with pytest.raises(oracle.OracleError):
        oracle.ancestors(parent)


@pytest.mark.parametrize("acc", [-2, 5, 99])
def test_invalid_accepted_rejected(acc):
    case = rand_case(81, B=1, N=5, Hk=1, Hv=1, dk=2, dv=2)
    with pytest.raises(oracle.OracleError):
        commit(case, np.array([acc], np.int32))


def test_gqa_consecutive_grouping():
    """value head h reads key head h // (Hv/Hk): with g = b = 0 only q matters"""
    case = rand_case(82, B=1, N=3, Hk=2, Hv=4, dk=3, dv=3)
    case["beta"][:] = 0.0
    case["g"][:] = 0.0
    o = verify(case)
    for h in range(4):
        np.testing.assert_allclose(o[0, :, h], case["q"][0, :, h // 2] @ case["S0"][0, h].T, rtol=1e-14)
