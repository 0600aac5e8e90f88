"""The gated-delta-rule commit oracle pinned to what the page and the
mathematics fix (flashinfer.gdn_decode.gated_delta_rule_replayssm_commit).

The page fixes: the accepted prefix of each request's cached windows is
committed in place; slots at or below null_block_id are ignored; a zero
accepted count is a no-op, tracking included; a tracked step outside the
accepted prefix leaves its destination unchanged; cached keys are
L2-normalised with epsilon 1e-6.  The delta rule S <- a S + b (v - a S k) k^T
fixes closed forms: b = 0 is pure decay exp(sum g) S0; with a = 1 and b = 1
the updated state maps the (unit) key to its value, S k = v; orthogonal unit
keys from S0 = 0 store their values, S = sum v_t k_t^T.  Normalised keys make
the result independent of the keys' scale; two commits chain into one.
"""
import numpy as np
import pytest

import rssm_inputs as ri

SMALL = ri.GdnSpec("gdn_pin", L=2, B=5, HV=4, H=2, T=6, slots=12, dk=8, dv=6, track=True)


def live_tiles(prob):
    """(b, layer, value head, slot, n, track slot or None, step) of every commit."""
    s = prob.spec
    out = []
    for b in range(s.B):
        slot, n = int(prob.state_indices[b]), int(prob.accept_lens[b])
        if slot <= s.null_block_id or n == 0:
            continue
        ts, step = None, -1
        if prob.track_state_indices is not None:
            t, st = int(prob.track_state_indices[b]), int(prob.track_steps[b])
            if t > s.null_block_id and 0 <= st < n:
                ts, step = t, st
        for l in range(s.L):
            for hv in range(s.HV):
                out.append((b, l, hv, slot, n, ts, step))
    return out


def keys(prob, l, slot, hv):
    """fp64 (T, dk) raw keys of the value head's key head."""
    import oracle
    s = prob.spec
    kh = hv // (s.HV // s.H)
    return oracle.decode("bf16", prob.rawk[l, slot, kh]).reshape(s.T, s.dk)


def values(prob, l, slot, hv):
    import oracle
    s = prob.spec
    return oracle.decode("bf16", prob.rawv[l, slot, hv]).reshape(s.T, s.dv)


def unit(k):
    return k / np.sqrt((k * k).sum(axis=-1, keepdims=True) + 1e-6)


def test_pure_decay_when_beta_zero(orc):
    prob = ri.make_gdn_problem(ri.with_(SMALL, accept=[6, 3, 1, 4, 2]), 60)
    prob.beta[:] = 0.0
    st0 = prob.state.copy()
    _, ex, _ = orc.gdn_commit(prob, want_exact=True)
    rows = live_tiles(prob)
    assert any(r[5] is not None for r in rows)
    for b, l, hv, slot, n, ts, step in rows:
        g = prob.g[l, slot, hv].astype(np.float64)
        np.testing.assert_allclose(ex[l, slot, hv], np.exp(g[:n].sum()) * st0[l, slot, hv], rtol=1e-12)
        if ts is not None:
            np.testing.assert_allclose(ex[l, ts, hv], np.exp(g[:step + 1].sum()) * st0[l, slot, hv], rtol=1e-12)


def test_delta_rule_stores_value_under_key(orc):
    """a = 1, b = 1: after token t the state maps the token's unit key to its
    value (the other directions keep their old images)."""
    spec = ri.with_(SMALL, B=1, L=1, HV=2, H=1)
    prob = ri.make_gdn_problem(spec, 61)
    prob.g[:] = 0.0
    prob.beta[:] = 1.0
    slot = int(prob.state_indices[0])
    for hv in range(spec.HV):
        k = unit(keys(prob, 0, slot, hv))
        v = values(prob, 0, slot, hv)
        for t in range(spec.T):
            _, _, S, _ = orc.gdn_tile(spec, prob.state[0, slot, hv], prob.rawk[0, slot, hv // 2],
                                      prob.rawv[0, slot, hv], prob.g[0, slot, hv], prob.beta[0, slot, hv],
                                      spec.T, track_step=t)
            np.testing.assert_allclose(S @ k[t], v[t], rtol=0, atol=1e-6 * (1 + np.abs(v[t]).max()))


def test_orthogonal_keys_store_their_values(orc):
    """S0 = 0 and mutually orthogonal keys: no key sees another's value, so
    S_n = sum_t beta_t (prod_{u>t} exp(g_u)) v_t k_t^T with unit keys
    k / sqrt(|k|^2 + 1e-6).  Decay comes before each update (the first
    token's value is not decayed by its own g), and one key is tiny
    (2^-10), where the epsilon's place inside the root shows."""
    spec = ri.with_(SMALL, B=1, L=1, HV=1, H=1, T=5, dk=8, dv=3)
    prob = ri.make_gdn_problem(spec, 62)
    slot = int(prob.state_indices[0])
    prob.state[:] = 0.0
    dirs = np.random.default_rng(63).permutation(spec.dk)[:spec.T]
    raw = np.zeros((spec.T, spec.dk), np.float32)
    mags = np.array([2.0, -0.5, 2.0 ** -10, 3.0, -1.0], np.float32)
    raw[np.arange(spec.T), dirs] = mags
    prob.rawk[0, slot, 0] = ri._bf16_codes(raw)
    g = prob.g[0, slot, 0].astype(np.float64)
    bt = prob.beta[0, slot, 0].astype(np.float64)
    for n in (1, 2, spec.T):
        S, _, _, _ = orc.gdn_tile(spec, prob.state[0, slot, 0], prob.rawk[0, slot, 0], prob.rawv[0, slot, 0],
                                  prob.g[0, slot, 0], prob.beta[0, slot, 0], n)
        v = values(prob, 0, slot, 0)
        k = unit(raw.astype(np.float64))
        want = sum(bt[t] * np.exp(g[t + 1:n].sum()) * np.outer(v[t], k[t]) for t in range(n))
        np.testing.assert_allclose(S, want, rtol=1e-12, atol=1e-15)
    assert abs(k[2, dirs[2]] - 2.0 ** -10 / np.sqrt(2.0 ** -20 + 1e-6)) < 1e-15


def test_normalised_keys_ignore_key_scale(orc):
    prob = ri.make_gdn_problem(SMALL, 64)
    _, ex, mg = orc.gdn_commit(prob, want_exact=True)
    prob4 = ri.make_gdn_problem(SMALL, 64)
    k = prob4.rawk.astype(np.uint32) << 16
    prob4.rawk = ri._bf16_codes(k.view(np.float32) * np.float32(4.0))   # exact in bf16
    _, ex4, _ = orc.gdn_commit(prob4, want_exact=True)
    w = ~np.isnan(ex)
    assert w.any()
    # only the epsilon sees the scale: relative key change <= 1e-6 / |k|^2
    assert (np.abs(ex4[w] - ex[w]) <= 1e-6 * mg[w]).all()
    # without normalisation the scale matters
    spec_raw = ri.with_(SMALL, use_l2norm=False)
    p1, p4 = ri.make_gdn_problem(spec_raw, 64), ri.make_gdn_problem(spec_raw, 64)
    p1.beta[:] = 0.01
    p4.beta[:] = 0.01
    p4.rawk = prob4.rawk
    _, e1, _ = orc.gdn_commit(p1, want_exact=True)
    _, e4, _ = orc.gdn_commit(p4, want_exact=True)
    assert not np.allclose(e1[w], e4[w], rtol=1e-3)


def test_key_head_grouping(orc):
    """Value head hv reads key head hv // (HV / H): zero keys on key head 0
    make value heads 0 and 1 pure decay, and heads 2 and 3 not."""
    prob = ri.make_gdn_problem(ri.with_(SMALL, accept=[6, 6, 6, 6, 6], null_frac=0.0), 65)
    prob.rawk[:, :, 0] = 0
    st0 = prob.state.copy()
    _, ex, _ = orc.gdn_commit(prob, want_exact=True)
    for b, l, hv, slot, n, ts, step in live_tiles(prob):
        decay = np.exp(prob.g[l, slot, hv].astype(np.float64)[:n].sum()) * st0[l, slot, hv]
        assert np.allclose(ex[l, slot, hv], decay, rtol=1e-12) == (hv < 2)


def test_two_commits_chain_into_one(orc):
    """Committing n1 tokens, then the next n2 (moved to the window's start),
    equals committing n1 + n2; the fp32 intermediate rounds by at most
    2^-24 M, and the update does not amplify it (|a| <= 1, |I - b k k^T| <= 1)."""
    spec = ri.with_(SMALL, track=False, null_frac=0.0)
    n1 = np.array([2, 1, 3, 0, 4])
    n2 = np.array([3, 5, 2, 6, 1])
    prob = ri.make_gdn_problem(ri.with_(spec, accept=list(n1 + n2)), 66)
    _, ex_direct, mg = orc.gdn_commit(prob, want_exact=True)
    p1 = ri.make_gdn_problem(ri.with_(spec, accept=list(n1)), 66)
    st1, _, _ = orc.gdn_commit(p1)
    p2 = ri.make_gdn_problem(ri.with_(spec, accept=list(n2)), 66)
    p2.state = st1
    for b in range(spec.B):
        s = int(prob.state_indices[b])
        a = int(n1[b])
        for arr, src in ((p2.rawv, prob.rawv), (p2.rawk, prob.rawk), (p2.g, prob.g), (p2.beta, prob.beta)):
            arr[:, s, :, :spec.T - a] = src[:, s, :, a:]
    _, ex2, _ = orc.gdn_commit(p2, want_exact=True)
    for b in range(spec.B):
        s = int(prob.state_indices[b])
        err = np.abs(ex2[:, s] - ex_direct[:, s])
        assert (err <= 2.0 ** -23 * mg[:, s] + 1e-300).all(), b


def test_noops_and_tracking_rules(orc):
    spec = ri.with_(SMALL, B=5, null_block_id=1, null_frac=0.0, accept=[0, 3, 3, 3, 6])
    prob = ri.make_gdn_problem(spec, 67)
    prob.state_indices[3] = 1                         # at null_block_id: ignored
    prob.track_steps[:] = [0, 3, -1, 1, 5]            # b1: step 3 >= n; b2: -1; b4: last token
    prob.track_state_indices[2] = 0                   # below null: also ignored
    out, ex, _ = orc.gdn_commit(prob, want_exact=True)
    written = np.zeros(prob.state.shape[:2], bool)
    for b, l, hv, slot, n, ts, step in live_tiles(prob):
        written[l, slot] = True
        if ts is not None:
            written[l, ts] = True
    # b0 accepts nothing (its track is not written either); b3's slot is null
    assert not written[:, prob.state_indices[0]].any() and not written[:, prob.track_state_indices[0]].any()
    assert not written[:, 1].any()
    # only b4 tracks; its track equals its final state bit for bit
    assert written[:, prob.track_state_indices[4]].all()
    for tb in (1, 2, 3):
        assert not written[:, prob.track_state_indices[tb]].any()
    np.testing.assert_array_equal(out[:, prob.track_state_indices[4]], out[:, prob.state_indices[4]])
    assert np.array_equal(out[~written], prob.state[~written])
    assert written.any()
