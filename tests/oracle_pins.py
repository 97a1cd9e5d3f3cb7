"""Pins that tie the CPU oracle to facts outside itself.

Each pin takes the oracle module as an argument, so the same checks can be run
against deliberately broken copies of the oracle (see test_oracle_mutants.py):
a plausible mistake anywhere in the oracle must make at least one pin fail.

Anchors used (none of them is the oracle's own formula retyped):
  * closed forms of tiny worked states (tests/golden/closed_forms.json);
  * a brute force that walks the page table page by page and accumulates the
    softmax in streaming form with scalar math;
  * torch's scaled_dot_product_attention and logsumexp in float64 on K/V gathered
    by plain indexing;
  * invariants the pages state: ⊕ is associative and commutative and splitting a
    key range then combining gives the unsplit state (Terms, "Attention State and
    ⊕"); the physical placement of pages does not change the result (Core
    mechanism 1); composed formats equal one plain format (Core mechanism 2);
  * limits and special cases: one key, identical keys, zero query, very large cap,
    GQA with replicated KV heads, causal first and last rows.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")
TIGHT = 1e-12


def _close(a, b, tol=TIGHT):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(diff)), "non-finite mismatch"
    assert np.all(diff <= tol * (1.0 + np.abs(np.where(both_inf, 0.0, b)))), float(np.max(diff))


# --------------------------------------------------------------------------- #
# Tiny page-table builders (independent of the input generators on purpose).
# --------------------------------------------------------------------------- #

def _layout(kv_logical, page_size, rng, pool_extra=2, permute=True):
    """Lay logical KV [B][l_kv, H, D] out into a paged pool; NaN in unused slots."""
    h_kv, d = kv_logical[0][0].shape[1], kv_logical[0][0].shape[2]
    n_pages = [(k.shape[0] + page_size - 1) // page_size for k, _ in kv_logical]
    total = sum(n_pages) + pool_extra
    order = rng.permutation(total) if permute else np.arange(total)
    k_pool = np.full((total, h_kv, page_size, d), np.nan)
    v_pool = np.full((total, h_kv, page_size, d), np.nan)
    kv_indptr = [0]
    kv_indices = []
    last = []
    nxt = 0
    for (k, v), n in zip(kv_logical, n_pages):
        pages = order[nxt : nxt + n]
        nxt += n
        for tau in range(k.shape[0]):
            k_pool[pages[tau // page_size], :, tau % page_size, :] = k[tau]
            v_pool[pages[tau // page_size], :, tau % page_size, :] = v[tau]
        kv_indices.extend(int(p) for p in pages)
        kv_indptr.append(kv_indptr[-1] + n)
        last.append(k.shape[0] - (n - 1) * page_size if n > 0 else page_size)
    return (
        k_pool,
        v_pool,
        np.asarray(kv_indptr, dtype=np.int32),
        np.asarray(kv_indices, dtype=np.int32),
        np.asarray(last, dtype=np.int32),
    )


def _random_case(rng, qo_lens, kv_lens, h_qo, h_kv, d, page_size, permute=True):
    q = rng.standard_normal((int(sum(qo_lens)), h_qo, d))
    kv = [
        (rng.standard_normal((l, h_kv, d)), rng.standard_normal((l, h_kv, d)))
        for l in kv_lens
    ]
    k_pool, v_pool, kv_indptr, kv_indices, last = _layout(kv, page_size, rng, permute=permute)
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32)
    return dict(
        q=q, kv=kv, k_pool=k_pool, v_pool=v_pool, qo_indptr=qo_indptr,
        kv_indptr=kv_indptr, kv_indices=kv_indices, last=last,
    )


def _run(O, c, page_size, h_qo, h_kv, scale, causal=False, cap=0.0):
    return O.bsr_attention(
        c["q"], c["k_pool"], c["v_pool"], c["qo_indptr"], c["kv_indptr"], c["kv_indices"],
        c["last"], page_size, h_qo, h_kv, scale, causal, cap,
    )


# --------------------------------------------------------------------------- #
# Brute force: a separate route through pages and the softmax.
# --------------------------------------------------------------------------- #

def brute_force(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, last, page_size,
                h_qo, h_kv, scale, causal, cap):
    """Walk each request's pages slot by slot; streaming softmax in scalar math."""
    total, _, d = q.shape
    g = h_qo // h_kv
    out = np.zeros((total, h_qo, v_pool.shape[3]))
    lse = np.full((total, h_qo), -math.inf)
    for r in range(len(qo_indptr) - 1):
        keys = []  # (kv_head-indexed rows) in logical order
        pages = kv_indices[kv_indptr[r] : kv_indptr[r + 1]]
        for pi, page in enumerate(pages):
            valid = page_size if pi < len(pages) - 1 else int(last[r])
            for slot in range(valid):
                keys.append((int(page), slot))
        l_kv = len(keys)
        l_qo = int(qo_indptr[r + 1] - qo_indptr[r])
        for t in range(l_qo):
            row = int(qo_indptr[r]) + t
            for h in range(h_qo):
                hk = h // g
                m = -math.inf
                z = 0.0
                acc = [0.0] * v_pool.shape[3]
                for j, (page, slot) in enumerate(keys):
                    if causal and j > l_kv - l_qo + t:
                        break
                    s = 0.0
                    for e in range(d):
                        s += float(q[row, h, e]) * float(k_pool[page, hk, slot, e])
                    s *= scale
                    if cap > 0:
                        s = cap * math.tanh(s / cap)
                    if s > m:
                        shrink = math.exp(m - s) if m > -math.inf else 0.0
                        z *= shrink
                        acc = [a * shrink for a in acc]
                        m = s
                    w = math.exp(s - m)
                    z += w
                    for e in range(len(acc)):
                        acc[e] += w * float(v_pool[page, hk, slot, e])
                if z > 0:
                    out[row, h] = [a / z for a in acc]
                    lse[row, h] = m + math.log(z)
    return out, lse


# --------------------------------------------------------------------------- #
# Pins
# --------------------------------------------------------------------------- #

def pin_closed_forms(O):
    """Golden worked states, placed in a 1-token-page pool at permuted pages."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        k = np.asarray(c["k"], dtype=np.float64)
        v = np.asarray(c["v"], dtype=np.float64)
        d = k.shape[1]
        k_pool = np.full((4, 1, 1, d), np.nan)
        v_pool = np.full((4, 1, 1, d), np.nan)
        pages = [3, 1]
        for j, p in enumerate(pages):
            k_pool[p, 0, 0] = k[j]
            v_pool[p, 0, 0] = v[j]
        q = np.asarray(c["q"], dtype=np.float64).reshape(1, 1, d)
        o, lse = O.bsr_attention(
            q, k_pool, v_pool, np.array([0, 1]), np.array([0, 2]), np.array(pages),
            np.array([1]), 1, 1, 1, c["scale"], False, c["cap"],
        )
        _close(o[0, 0], c["o"], 1e-14)
        _close(lse[0, 0], c["lse"], 1e-14)


def pin_merge_worked(O):
    """The two-key state equals the ⊕ of its one-key states ((1,0), 1) and ((0,1), 0)."""
    with open(GOLDEN) as f:
        c = json.load(f)["cases"][0]
    o, lse = O.merge_state(
        np.array([[1.0, 0.0]]), np.array([1.0]), np.array([[0.0, 1.0]]), np.array([0.0])
    )
    _close(o[0], c["o"], 1e-15)
    _close(lse[0], c["lse"], 1e-15)
    # order-swapped and with the identity state
    o2, lse2 = O.merge_state(
        np.array([[0.0, 1.0]]), np.array([0.0]), np.array([[1.0, 0.0]]), np.array([1.0])
    )
    _close(o2[0], c["o"], 1e-15)
    o3, lse3 = O.merge_state(o, lse, np.zeros((1, 2)), np.array([-np.inf]))
    _close(o3, o, 0)
    _close(lse3, lse, 0)
    o4, lse4 = O.merge_state(np.zeros((1, 2)), np.array([-np.inf]), np.zeros((1, 2)), np.array([-np.inf]))
    assert np.all(o4 == 0) and np.all(np.isneginf(lse4))


def pin_brute_force(O):
    rng = np.random.default_rng(11)
    shapes = [
        # qo_lens, kv_lens, h_qo, h_kv, d, P, causal, cap
        ([1, 1, 1], [5, 1, 9], 4, 2, 4, 3, False, 0.0),
        ([1, 2], [7, 16], 2, 2, 8, 16, False, 5.0),
        ([3, 2, 1], [3, 7, 4], 4, 1, 4, 2, True, 0.0),
        ([4, 1], [9, 6], 8, 2, 4, 1, True, 3.0),
        ([2, 1], [0, 3], 2, 1, 4, 2, False, 0.0),
    ]
    for qo, kv, h_qo, h_kv, d, P, causal, cap in shapes:
        c = _random_case(rng, qo, kv, h_qo, h_kv, d, P)
        scale = 0.37
        o, lse = _run(O, c, P, h_qo, h_kv, scale, causal, cap)
        ob, lb = brute_force(
            c["q"], c["k_pool"], c["v_pool"], c["qo_indptr"], c["kv_indptr"], c["kv_indices"],
            c["last"], P, h_qo, h_kv, scale, causal, cap,
        )
        _close(o, ob)
        _close(lse, lb)


def pin_sdpa(O):
    """float64 torch scaled_dot_product_attention and logsumexp on gathered K/V."""
    rng = np.random.default_rng(12)
    for qo, kv, h_qo, h_kv, d, P, causal in [
        ([1, 1, 1, 1], [17, 64, 100, 255], 8, 2, 64, 16, False),
        ([6, 5], [6, 5], 4, 4, 8, 3, True),      # no cached prefix: top-left == bottom-right
        ([3, 4], [10, 4], 4, 2, 16, 2, True),    # cached prefix: explicit bottom-right mask
        ([5], [12], 8, 1, 32, 4, False),
    ]:
        c = _random_case(rng, qo, kv, h_qo, h_kv, d, P)
        scale = 1.0 / math.sqrt(d)
        o, lse = _run(O, c, P, h_qo, h_kv, scale, causal)
        g = h_qo // h_kv
        for r, (k, v) in enumerate(c["kv"]):
            q0, q1 = int(c["qo_indptr"][r]), int(c["qo_indptr"][r + 1])
            qt = torch.from_numpy(c["q"][q0:q1]).permute(1, 0, 2)  # [H, l_qo, D]
            kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)
            vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
            l_qo, l_kv = q1 - q0, k.shape[0]
            if causal and l_qo == l_kv:
                ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
                mask = torch.ones(l_qo, l_kv, dtype=torch.bool).tril()
            else:
                mask = torch.ones(l_qo, l_kv, dtype=torch.bool)
                if causal:
                    mask = mask.tril(diagonal=l_kv - l_qo)
                ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
            scores = torch.matmul(qt, kt.transpose(1, 2)) * scale
            scores = scores.masked_fill(~mask, float("-inf"))
            ref_lse = torch.logsumexp(scores, dim=-1)
            _close(o[q0:q1], ref.permute(1, 0, 2).numpy(), 1e-12)
            _close(lse[q0:q1], ref_lse.permute(1, 0).numpy(), 1e-12)


def pin_special_cases(O):
    rng = np.random.default_rng(13)
    d = 8
    # a single key: O = v0 and LSE = s0
    c = _random_case(rng, [1], [1], 2, 1, d, 4)
    o, lse = _run(O, c, 4, 2, 1, 0.5)
    k, v = c["kv"][0]
    _close(o[0, 0], v[0, 0])
    _close(lse[0, 0], 0.5 * float(c["q"][0, 0] @ k[0, 0]))
    # identical keys: O = mean(V), LSE = s + ln L, with L = 8192 -> ln L = 9.010913347279288
    L = 8192
    kk = np.tile(rng.standard_normal((1, 1, d)), (L, 1, 1))
    vv = rng.standard_normal((L, 1, d))
    k_pool, v_pool, kv_indptr, kv_indices, last = _layout([(kk, vv)], 16, rng)
    q = rng.standard_normal((1, 1, d))
    o, lse = O.bsr_attention(q, k_pool, v_pool, np.array([0, 1]), kv_indptr, kv_indices, last, 16, 1, 1, 0.25)
    _close(o[0, 0], vv[:, 0].mean(axis=0), 1e-12)
    _close(lse[0, 0], 0.25 * float(q[0, 0] @ kk[0, 0]) + 9.010913347279288, 1e-12)
    # zero query: O = mean(V), LSE = ln L, for any cap
    q0 = np.zeros((1, 1, d))
    for cap in (0.0, 2.0):
        o, lse = O.bsr_attention(q0, k_pool, v_pool, np.array([0, 1]), kv_indptr, kv_indices, last, 16, 1, 1, 0.25, False, cap)
        _close(o[0, 0], vv[:, 0].mean(axis=0), 1e-12)
        _close(lse[0, 0], math.log(L), 1e-12)
    # a huge cap is no cap
    c = _random_case(rng, [2], [9], 2, 1, d, 3)
    a = _run(O, c, 3, 2, 1, 0.3, False, 0.0)
    b = _run(O, c, 3, 2, 1, 0.3, False, 1e30)
    _close(a[0], b[0], 1e-12)
    _close(a[1], b[1], 1e-12)
    # empty request: O = 0, LSE = -inf
    c = _random_case(rng, [1, 1], [0, 5], 2, 1, d, 2)
    o, lse = _run(O, c, 2, 2, 1, 0.3)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


def pin_causal_rows(O):
    """Causal, bottom-right: the first new token of a request with prefix p sees p+1 keys, the last sees all."""
    rng = np.random.default_rng(14)
    d = 4
    for prefix in (0, 5):
        l_qo = 3
        c = _random_case(rng, [l_qo], [prefix + l_qo], 1, 1, d, 2)
        o, lse = _run(O, c, 2, 1, 1, 0.7, True)
        k, v = c["kv"][0]
        q = c["q"]
        # first row over keys 0..prefix, from the textbook softmax with math.fsum
        s = [0.7 * float(q[0, 0] @ k[j, 0]) for j in range(prefix + 1)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        _close(lse[0, 0], m + math.log(z))
        _close(o[0, 0], [math.fsum(w[j] * v[j, 0, e] for j in range(prefix + 1)) / z for e in range(d)])
        if prefix == 0:
            _close(o[0, 0], v[0, 0])
        # last row sees everything: equals the non-causal result
        o_nc, lse_nc = _run(O, c, 2, 1, 1, 0.7, False)
        _close(o[l_qo - 1], o_nc[l_qo - 1])
        _close(lse[l_qo - 1], lse_nc[l_qo - 1])


def pin_page_layout_invariance(O):
    """Same logical KV, different page sizes and physical placement: identical bits."""
    rng = np.random.default_rng(15)
    qo, kv, h_qo, h_kv, d = [1, 2, 1], [23, 5, 16], 4, 2, 8
    q = rng.standard_normal((sum(qo), h_qo, d))
    logical = [(rng.standard_normal((l, h_kv, d)), rng.standard_normal((l, h_kv, d))) for l in kv]
    qo_indptr = np.concatenate([[0], np.cumsum(qo)])
    ref = None
    for P in (1, 2, 3, 16):
        for permute in (False, True):
            k_pool, v_pool, kv_indptr, kv_indices, last = _layout(logical, P, rng, permute=permute)
            o, lse = O.bsr_attention(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.3, False, 0.0)
            if ref is None:
                ref = (o, lse)
            else:
                assert np.array_equal(o, ref[0]) and np.array_equal(lse, ref[1])
    # and the page walk reads what was laid out: compare with a dense run on the logical rows
    for r, (k, v) in enumerate(logical):
        for h in range(h_qo):
            s = 0.3 * (q[qo_indptr[r]:qo_indptr[r + 1], h] @ k[:, h // (h_qo // h_kv)].T)
            ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
            _close(ref[1][qo_indptr[r]:qo_indptr[r + 1], h], ref_lse)


def pin_gqa(O):
    """GQA equals MHA over KV heads replicated g times (query head h reads KV head h // g)."""
    rng = np.random.default_rng(16)
    h_qo, h_kv, d, P = 8, 2, 8, 4
    g = h_qo // h_kv
    c = _random_case(rng, [1, 3], [9, 6], h_qo, h_kv, d, P)
    o, lse = _run(O, c, P, h_qo, h_kv, 0.4)
    rep = dict(c)
    rep["k_pool"] = np.repeat(c["k_pool"], g, axis=1)
    rep["v_pool"] = np.repeat(c["v_pool"], g, axis=1)
    o2, lse2 = _run(O, rep, P, h_qo, h_qo, 0.4)
    _close(o, o2, 0)
    _close(lse, lse2, 0)
    # g = 1 with a single head reduces to plain single-head attention
    c1 = _random_case(rng, [2], [5], 1, 1, d, P)
    o1, lse1 = _run(O, c1, P, 1, 1, 0.4)
    k, v = c1["kv"][0]
    s = 0.4 * (c1["q"][:, 0] @ k[:, 0].T)
    w = torch.softmax(torch.from_numpy(s), dim=-1).numpy()
    _close(o1[:, 0], w @ v[:, 0])


def pin_merge_invariants(O):
    """Split at any point then ⊕ equals unsplit; ⊕ is associative and commutative."""
    rng = np.random.default_rng(17)
    d = 6
    for L in (2, 7, 40):
        q = rng.standard_normal((3, d))
        k = rng.standard_normal((L, d))
        v = rng.standard_normal((L, d))
        full = O.attention_dense(q, k, v, 0.5, 4.0)
        for a in (1, L // 2, L - 1):
            left = O.attention_dense(q, k[:a], v[:a], 0.5, 4.0)
            right = O.attention_dense(q, k[a:], v[a:], 0.5, 4.0)
            m = O.merge_state(left[0], left[1], right[0], right[1])
            _close(m[0], full[0])
            _close(m[1], full[1])
            m2 = O.merge_state(right[0], right[1], left[0], left[1])
            _close(m2[0], full[0])
            _close(m2[1], full[1])
        cuts = sorted({1, L // 3, 2 * L // 3, L - 1} - {0})
        parts = []
        prev = 0
        for ct in cuts + [L]:
            if ct > prev:
                parts.append(O.attention_dense(q, k[prev:ct], v[prev:ct], 0.5, 4.0))
                prev = ct
        fold = O.merge_states(parts)
        _close(fold[0], full[0])
        _close(fold[1], full[1])
        if len(parts) >= 3:
            right_assoc = O.merge_state(parts[0][0], parts[0][1], *O.merge_state(parts[1][0], parts[1][1], parts[2][0], parts[2][1]))
            left_assoc = O.merge_state(*O.merge_state(parts[0][0], parts[0][1], parts[1][0], parts[1][1]), parts[2][0], parts[2][1])
            _close(right_assoc[0], left_assoc[0])
            _close(right_assoc[1], left_assoc[1])


def pin_composable(O):
    """A shared-prefix block row plus per-branch suffix rows equals one plain format."""
    rng = np.random.default_rng(18)
    branches, h_qo, h_kv, d, P = 5, 4, 2, 8, 4
    prefix_len = 12  # whole pages
    suf = [3, 9, 4, 1, 6]
    pre = (rng.standard_normal((prefix_len, h_kv, d)), rng.standard_normal((prefix_len, h_kv, d)))
    sufs = [(rng.standard_normal((s, h_kv, d)), rng.standard_normal((s, h_kv, d))) for s in suf]
    k_pool, v_pool, ip, idx, last = _layout([pre] + sufs, P, rng)
    n_pre = ip[1]
    q = rng.standard_normal((branches, h_qo, d))
    formats = [
        dict(qo_indptr=np.array([0, branches]), kv_indptr=np.array([0, n_pre]), last_page_len=last[:1], kv_indices_offset=0),
        dict(qo_indptr=np.arange(branches + 1), kv_indptr=ip[1:] - n_pre, last_page_len=last[1:], kv_indices_offset=int(n_pre)),
    ]
    oc, lc = O.composable_attention(q, k_pool, v_pool, formats, idx, P, h_qo, h_kv, 0.3, 2.0)
    single_idx, single_ip = [], [0]
    for b in range(branches):
        pages = list(idx[: n_pre]) + list(idx[ip[b + 1] : ip[b + 2]])
        single_idx += pages
        single_ip.append(single_ip[-1] + len(pages))
    os_, ls = O.bsr_attention(
        q, k_pool, v_pool, np.arange(branches + 1), np.array(single_ip), np.array(single_idx),
        last[1:], P, h_qo, h_kv, 0.3, False, 2.0,
    )
    _close(oc, os_)
    _close(lc, ls)
    # and the ⊕ of the per-format states gives the same
    op, lp = O.bsr_attention(q, k_pool, v_pool, np.array([0, branches]), np.array([0, n_pre]), idx, last[:1], P, h_qo, h_kv, 0.3, False, 2.0)
    osu, lsu = O.bsr_attention(q, k_pool, v_pool, np.arange(branches + 1), ip[1:], idx, last[1:], P, h_qo, h_kv, 0.3, False, 2.0)
    om, lm = O.merge_state(op, lp, osu, lsu)
    _close(om, os_)
    _close(lm, ls)


ALL_PINS = [
    pin_closed_forms,
    pin_merge_worked,
    pin_brute_force,
    pin_sdpa,
    pin_special_cases,
    pin_causal_rows,
    pin_page_layout_invariance,
    pin_gqa,
    pin_merge_invariants,
    pin_composable,
]
