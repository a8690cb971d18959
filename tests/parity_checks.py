"""Comparison helpers shared by the GPU parity tests (no test of its own)."""
import numpy as np

TIE_BAND = 1e-5


def check_labels_in_tie_band(X, C, lab, a, max_share):
    """GPU labels against the oracle's assignment ``a`` of X to C: equal for
    every token whose margin is at least TIE_BAND; the excluded tokens are at
    most ``max_share`` of the tokens, and for each of them the GPU's centroid is
    within the band of the nearest one:
    (||x - c_gpu||^2 - ||x - c_best||^2) / (||x||^2 + ||c_best||^2) < TIE_BAND."""
    clear = a.margin >= TIE_BAND
    share = float(np.mean(~clear))
    print(f"tie band: {int((~clear).sum())} of {len(lab)} tokens ({share:.2e})", flush=True)
    assert share <= max_share
    np.testing.assert_array_equal(lab[clear], a.labels[clear])
    ex = np.nonzero(~clear)[0]
    if len(ex):
        x = X[ex]
        best = C[a.labels[ex]]
        d_best = np.sum((x - best) ** 2, axis=1)
        d_gpu = np.sum((x - C[lab[ex]]) ** 2, axis=1)
        rel = (d_gpu - d_best) / (np.sum(x * x, axis=1) + np.sum(best * best, axis=1))
        assert np.all(rel < TIE_BAND * (1 + 1e-9)), float(rel.max())
