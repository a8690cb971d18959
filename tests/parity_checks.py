"""Comparison helpers shared by the GPU parity tests (no test of its own)."""
import numpy as np

# The GPU decides every assignment exactly: matrix-core distances settle the
# tokens whose two nearest centroids are further apart than the proven error
# of those distances, and the rest are decided again in fp64.  GPU and oracle
# (fp64, expanded form) can then differ only where the relative margin is at
# the level of fp64 rounding, far below this band.
TIE_BAND = 1e-12


def check_labels_in_tie_band(X, C, lab, a, max_share, band=TIE_BAND):
    """GPU labels against the oracle's assignment ``a`` of X to C: equal for
    every token whose margin is at least ``band``; the excluded tokens are at
    most ``max_share`` of the tokens, and for each of them the GPU's centroid is
    within the band of the nearest one:
    (||x - c_gpu||^2 - ||x - c_best||^2) / (||x||^2 + ||c_best||^2) < band."""
    clear = a.margin >= band
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
        assert np.all(rel < band * (1 + 1e-9) + 1e-15), float(rel.max())
