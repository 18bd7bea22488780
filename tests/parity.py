"""Comparison rules between the GPU layer and the CPU oracle (test helpers).

Routing: top-k ids must match the oracle's set exactly for every token whose
top-k margin (k-th minus (k+1)-th oracle fp32 logit) exceeds 1e-4.  On a
near-tie the GPU may pick differently, but only among experts within 1e-4 of
the k-th logit.  Layer output: max|y - y_oracle| <= 2e-2 * RMS(y_oracle), where
the oracle recomputes the near-tie tokens under the GPU's own routing.  The
bars (MARGIN, WEIGHT_TOL, Y_TOL) live in tests/tolerances.py and are derived in
tests/test_tolerances.py.
"""
import numpy as np

import oracle
from tests.tolerances import MARGIN, WEIGHT_TOL, Y_TOL  # noqa: F401


def check_routing(ids_gpu, w_gpu, ids_or, p_or, margin, logits, k):
    """Returns the list of tokens whose GPU expert set legitimately differs.
    Raises AssertionError on any illegal difference."""
    ids_gpu = np.asarray(ids_gpu)
    w_gpu = np.asarray(w_gpu, np.float64)
    T = ids_gpu.shape[0]
    flipped = []
    # weights: a probability vector per token, close to the oracle's when the sets match
    assert np.all(np.abs(w_gpu.sum(1) - 1.0) <= 1e-6 * k), "GPU weights do not sum to 1"
    assert np.all(w_gpu >= 0)
    for t in range(T):
        sg = set(ids_gpu[t].tolist())
        so = set(ids_or[t].tolist())
        assert len(sg) == k, "token %d: repeated expert ids %s" % (t, ids_gpu[t])
        if sg == so:
            # same set: slot weights must agree per expert id
            pg = dict(zip(ids_gpu[t].tolist(), w_gpu[t].tolist()))
            po = dict(zip(ids_or[t].tolist(), p_or[t].tolist()))
            for e in so:
                assert abs(pg[e] - po[e]) <= WEIGHT_TOL, "token %d expert %d: weight %g vs %g" % (
                    t, e, pg[e], po[e])
            continue
        assert margin[t] <= MARGIN, "token %d: ids %s vs oracle %s at margin %g" % (
            t, sorted(sg), sorted(so), margin[t])
        l = logits[t].astype(np.float64)
        lk = np.sort(l)[::-1][k - 1]
        must = {e for e in range(l.size) if l[e] > lk + MARGIN}
        assert must <= sg, "token %d: dropped a clear winner" % t
        assert all(l[e] >= lk - MARGIN for e in sg), "token %d: chose a clear loser" % t
        flipped.append(t)
    return flipped


def reference_y(inp, ids_or, p_or, ids_gpu, w_gpu, flipped, tokens):
    """Oracle y for ``tokens``; tokens in ``flipped`` use the GPU's routing."""
    ids = np.array(ids_or, np.int32, copy=True)
    p = np.array(p_or, np.float64, copy=True)
    for t in flipped:
        ids[t] = ids_gpu[t]
        p[t] = w_gpu[t]
    return oracle.experts(inp, ids, p, tokens=np.asarray(tokens, np.int64))


def y_error(y_gpu, y_ref):
    """max|err| / RMS(y_ref)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    rms = float(np.sqrt(np.mean(np.square(y_ref))))
    err = float(np.max(np.abs(y_gpu - y_ref))) if y_ref.size else 0.0
    return err / rms if rms > 0 else err, err, rms


def sample_tokens(T, n, extra=()):
    """Deterministic subset: every (T/n)-th token, the last token, plus extra."""
    step = max(1, T // max(n, 1))
    s = set(range(0, T, step)) | {T - 1} | {int(t) for t in extra if 0 <= t < T}
    return np.array(sorted(s), np.int64)


def tile_edge_tokens(ref, bm):
    """Tokens owning the first and the last valid row of every m-tile of every
    group, with the rows of an m-tile as the grouped GEMMs cut them: BM rows
    each, except that with 256-row tiles a group of exactly two m-tiles shares
    its rows out evenly (ceil(count / 2) rounded up to 32 rows per m-tile).
    ``ref`` is an oracle.align result (row_token maps a padded row to its token)."""
    toks = set()
    counts, padded, row_token = ref["counts"], ref["padded"], ref["row_token"]
    for g in range(counts.size):
        cnt, p0 = int(counts[g]), int(padded[g])
        if cnt == 0:
            continue
        mg = (int(padded[g + 1]) - p0) // bm
        q = ((cnt + 1) // 2 + 31) // 32 * 32 if (bm == 256 and mg == 2) else bm
        for j in range(-(-cnt // q)):
            for r in (j * q, min((j + 1) * q, cnt) - 1):
                toks.add(int(row_token[p0 + r]))
    return sorted(toks)


def align_equal(gpu, ref):
    """Bit-exact comparison of a GPU moe_align result with oracle.align."""
    G = ref["counts"].size
    nt = int(gpu["n_tiles"][0])
    assert nt == ref["n_tiles"], "n_tiles %d vs %d" % (nt, ref["n_tiles"])
    for key in ("counts", "offsets", "padded", "sorted_assign", "row_of"):
        g = np.asarray(gpu[key])[:ref[key].size]
        assert np.array_equal(g, ref[key]), "%s differs" % key
    rows = int(ref["padded"][G])
    assert np.array_equal(np.asarray(gpu["row_token"])[:rows], ref["row_token"]), "row_token differs"
    assert np.array_equal(np.asarray(gpu["tile_group"])[:nt], ref["tile_group"]), "tile_group differs"
