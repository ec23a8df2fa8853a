"""Element-by-element comparison of a GPU layer call with the oracle.

What must match exactly (unique results): router ids away from near-ties, the
permutation, the quantized activations of the 8/4-bit modes (bf16 inputs, so
the fp32 quantizer steps are identical on both sides), and every code of the
intermediate h away from rounding midpoints.  What may differ (several correct
results): router ids at logits closer than the fp32 accumulation error of the
logit sums (the pages note that a rounding difference can change which experts
the router picks: page "Infernix", section "Quality"), and codes of h at
midpoints (tests/ties.py).  Tolerances:

* routing weights: 1e-5 absolute; sum of a token's weights within 4 k 2^-24 of 1;
* per pair, the down projection y: relative L2 error <= 1e-4 against the
  oracle's double result for the same intermediate (fp32 accumulation only);
* per token, the bf16 output: ||out - bf16(oracle)||_2 <= 2e-3 ||bf16(oracle)||_2,
  where bf16(oracle) is the double result rounded once.  The element-wise
  relative error cannot meet 2e-3 for any correct bf16 output (rounding alone
  reaches 2^-8), so the per-row L2 norm carries the bound.  It is checked twice:
  against the oracle continued from the GPU's (validated) intermediate codes,
  and against the oracle's own nominal result -- for every token in the 16-bit
  modes (a flipped bf16 or fp16 code of h moves the output by ~10^-4), and in
  the 8- and 4-bit modes for every token none of whose pairs flipped a code
  (one E4M3 step is up to 1/8 of an element, one E2M1 step up to 1/2: a flip can
  move a token's output by 10^-3 .. 10^-2, several correct results).
* flipped intermediate codes: at most tests/ties.py's budget (a fraction of the
  elements whose window admits two codes).
"""
from __future__ import annotations

import numpy as np

from oracle import formats as F
from oracle import layer as OL
from tests import ties

OUT_TOL = 2e-3
Y_TOL = 1e-4
W_TOL = 1e-5
LOGIT_WINDOW = 2.0 ** -20


def route_window(x_u16, wr_u16):
    """Per-token bound on fp32-vs-double logit differences: 2^-20 max_e sum_h |x_h Wr[e,h]|."""
    ax = np.abs(F.bf16_to_f64(x_u16))
    aw = np.abs(F.bf16_to_f64(wr_u16))
    return LOGIT_WINDOW * (ax @ aw.T).max(axis=1)


def check_route(x_u16, wr_u16, bias, k, ids_gpu, w_gpu):
    """Returns (oracle Route, list of tokens where the GPU took another valid choice)."""
    r = OL.route(x_u16, wr_u16, k, bias)
    delta = route_window(x_u16, wr_u16)
    T = ids_gpu.shape[0]
    flipped = []
    for t in range(T):
        g = ids_gpu[t].astype(np.int64)
        l = r.logits[t]
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < l.size, (t, g)
        if not np.array_equal(g, r.ids[t]):
            kth = np.sort(l)[::-1][k - 1]
            must = np.nonzero(l > kth + delta[t])[0]
            may = np.nonzero(l >= kth - delta[t])[0]
            assert set(must.tolist()) <= set(g.tolist()) <= set(may.tolist()), \
                f"token {t}: GPU ids {g} are not a valid top-{k} (window {delta[t]:.3g})"
            assert np.all(l[g[:-1]] >= l[g[1:]] - delta[t]), f"token {t}: order {g}"
            flipped.append(t)
        le = l[g]
        ex = np.exp(le - le.max())
        w_exp = ex / ex.sum()
        assert np.max(np.abs(w_gpu[t] - w_exp)) <= W_TOL, (t, w_gpu[t], w_exp)
        assert abs(float(np.sum(w_gpu[t].astype(np.float64))) - 1.0) <= 4 * k * 2.0 ** -24
    return r, flipped


def check_permutation(ids_gpu, E, offsets, sorted_pairs, pair_row, oracle_ids=None):
    """Exact against the oracle's permutation when the ids agree; otherwise the
    stable-counting-sort properties of the GPU's own ids."""
    if oracle_ids is not None and np.array_equal(ids_gpu, oracle_ids):
        p = OL.permute(oracle_ids, E)
        assert np.array_equal(offsets, p.offsets)
        assert np.array_equal(sorted_pairs, p.sorted_pairs)
        assert np.array_equal(pair_row, p.pair_row)
        return
    flat = ids_gpu.reshape(-1).astype(np.int64)
    cnt = np.bincount(flat, minlength=E)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(cnt)]))
    assert np.array_equal(np.sort(sorted_pairs), np.arange(flat.size))
    for e in range(E):
        seg = sorted_pairs[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    assert np.array_equal(pair_row[sorted_pairs], np.arange(flat.size))


def check_experts(w, mode, x_u16, get_expert, k, offsets, sorted_pairs, y_gpu, ffn_ws, tokens=None,
                  report=None):
    """Per expert segment: the activation quantization (exact), the intermediate
    (ties.py rules) and y (relative L2 per pair).  Returns y_expected [P, H] (NaN
    rows where not checked) and a dict of counts."""
    rep = report if report is not None else ties.TieReport()
    P, H = y_gpu.shape
    y_exp = np.full((P, H), np.nan)
    y_nom = np.full((P, H), np.nan)
    row_flipped = np.zeros(P, bool)
    E = offsets.size - 1
    worst = 0.0
    for e in np.nonzero(np.diff(offsets))[0]:
        rows = np.arange(offsets[e], offsets[e + 1])
        toks = sorted_pairs[rows] // k
        if tokens is not None:
            keep = np.isin(toks, tokens)
            rows, toks = rows[keep], toks[keep]
            if rows.size == 0:
                continue
        ex = get_expert(int(e))
        res = OL.expert_ffn(ex, x_u16[toks], mode)
        # activations as the kernels store them: unique, so exact
        if mode == "A8":
            c, s = OL.quantize_activation(F.bf16_to_f64(x_u16[toks]).astype(np.float32), "A8")[0]
            assert np.array_equal(ffn_ws["x_codes"][toks], c)
            assert np.array_equal(ffn_ws["x_scales"][toks], s)
        elif mode == "A4":
            for m in (0, 1):
                c, s = OL.quantize_activation(F.bf16_to_f64(x_u16[toks]).astype(np.float32), "A4",
                                              ex.gu_inscale[m])[0]
                assert np.array_equal(ffn_ws["x_codes"][rows, m], c), (e, m)
                assert np.array_equal(ffn_ws["x_scales"][rows, m], s), (e, m)
        if mode in ("A16", "F16"):
            gpu_h = ffn_ws["h"][rows]
        else:
            gpu_h = (ffn_ws["h_codes"][rows], ffn_ws["h_scales"][rows])
        hdq = ties.expected_intermediate(res, mode, gpu_h, ex.dn_inscale, rep)
        row_flipped[rows] = rep.row_flips
        y = hdq @ ex.down().T
        y_exp[rows] = y
        y_nom[rows] = res.y
        err = np.linalg.norm(y_gpu[rows] - y, axis=1) / np.maximum(np.linalg.norm(y, axis=1), 1e-30)
        worst = max(worst, float(err.max()))
        assert err.max() <= Y_TOL, f"expert {e}: y rel err {err.max():.3g}"
    rep.check()
    return y_exp, {"y_worst_rel": worst, "ties": repr(rep), "y_nominal": y_nom, "row_flipped": row_flipped,
                   "tie_two_candidate": rep.two_candidate, "tie_flipped": rep.flipped}


def _weighted(y, route_oracle, ids, pair_row, t, k):
    l = route_oracle.logits[t][ids[t]]
    ex = np.exp(l - l.max())
    wt = ex / ex.sum()
    acc = np.zeros(y.shape[1])
    for j in range(k):
        acc += wt[j] * y[pair_row[t * k + j]]
    return acc


def _rel_l2(got, acc):
    ref = F.bf16_to_f64(F.f64_to_bf16(acc))
    return np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)


def check_shared(sh, x_u16, h_gpu, y_gpu, report=None):
    """The shared expert's stored bf16 intermediate (tests/ties.py rules, as the
    16-bit mode's) and its gated output y (relative L2 per token <= Y_TOL against
    the oracle continued from the GPU's validated intermediate).  Returns (that
    expected gated y [T, H], the oracle's SharedResult, info)."""
    rep = report if report is not None else ties.TieReport()
    res = OL.shared_expert(sh, x_u16)
    hdq = ties.expected_intermediate(res, "A16", h_gpu, None, rep)
    rep.check()
    y = res.sig[:, None] * (hdq @ F.bf16_to_f64(sh.dn).T)
    err = np.linalg.norm(y_gpu - y, axis=1) / np.maximum(np.linalg.norm(y, axis=1), 1e-30)
    assert err.max() <= Y_TOL, f"shared expert y rel err {err.max():.3g}"
    return y, res, {"shared_y_worst_rel": float(err.max()), "shared_ties": repr(rep),
                    "shared_flipped_rows": rep.row_flips}


def check_output(out_gpu_u16, y_exp, pair_row, route_oracle, ids_gpu, k, tokens=None, mode=None, y_nom=None,
                 row_flipped=None, oracle_ids=None, shared_exp=None, shared_nom=None):
    """Per token rel-L2 of the bf16 output against bf16(oracle double result): the
    oracle continued from the GPU's validated intermediate (y_exp), and, where the
    GPU made no other valid choice (same routing; in the 4-bit mode also no flipped
    intermediate code), the oracle's own nominal result (y_nom).  With a shared
    expert, its gated output (shared_exp: continued from the GPU's intermediate;
    shared_nom: the oracle's own) joins the sum before the rounding."""
    T = out_gpu_u16.shape[0]
    toks = range(T) if tokens is None else tokens
    worst, inf_worst, within_ulp, nom_worst, nom_n = 0.0, 0.0, [], 0.0, 0
    for t in toks:
        acc = _weighted(y_exp, route_oracle, ids_gpu, pair_row, t, k)
        if shared_exp is not None:
            acc = acc + shared_exp[t]
        got = F.bf16_to_f64(out_gpu_u16[t])
        rel = _rel_l2(got, acc)
        worst = max(worst, rel)
        inf_worst = max(inf_worst, float(np.max(np.abs(got - acc)) / max(np.max(np.abs(acc)), 1e-30)))
        ulp = np.abs(acc) * 2.0 ** -7 + 1e-38
        within_ulp.append(float(np.mean(np.abs(got - acc) <= ulp)))
        assert rel <= OUT_TOL, f"token {t}: rel L2 {rel:.3g}"
        if y_nom is None:
            continue
        same_route = oracle_ids is None or np.array_equal(ids_gpu[t], oracle_ids[t])
        rows = pair_row[t * k:(t + 1) * k]
        if same_route and (mode not in ("A4", "A8") or not np.any(row_flipped[rows])):
            acc_n = _weighted(y_nom, route_oracle, ids_gpu, pair_row, t, k)
            if shared_nom is not None:
                acc_n = acc_n + shared_nom[t]
            rel_n = _rel_l2(got, acc_n)
            nom_worst = max(nom_worst, rel_n)
            nom_n += 1
            assert rel_n <= OUT_TOL, f"token {t}: rel L2 {rel_n:.3g} against the oracle's nominal result"
    return {"out_worst_rel_l2": worst, "out_inf_rel_vs_double": inf_worst,
            "frac_within_1ulp": float(np.mean(within_ulp)),
            "out_vs_nominal_worst_rel_l2": nom_worst, "tokens_vs_nominal": nom_n}
