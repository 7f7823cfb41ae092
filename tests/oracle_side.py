"""Test-side glue: feeds the synthetic workloads' bytes to the float64 oracle and
compares GPU results with it (certified top-k rows, tolerances)."""
import numpy as np

from oracle import lca_oracle as O
from oracle.workloads import LazyRows, oracle_decode, oracle_decode_state, oracle_prefill  # noqa: F401


# ---------------------------------------------------------------------------
# comparisons


def ulp_of(x, fmt):
    """One unit in the last place of the stored format at |x| (float64)."""
    x = np.abs(np.asarray(x, np.float64))
    mb = {"bf16": 7, "fp8": 3, "f32": 23}[fmt]
    emin = {"bf16": -126, "fp8": -6, "f32": -126}[fmt]
    _, E = np.frexp(np.maximum(x, 1e-300))
    return np.exp2(np.maximum(E - 1, emin) - mb)


def assert_within_ulp(got, want, fmt, n_ulp=1.0, slack=None, what=""):
    """Stored values: |got - want| <= n_ulp ulp of the format (per dim for the mixed
    KV) plus `slack`, the oracle's bound on the fp32 evaluation error before the
    cast (it matters only near zero, where cancellation makes an ulp tiny)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    sl = np.zeros_like(want) if slack is None else np.broadcast_to(np.asarray(slack, np.float64), want.shape)
    if fmt == "fp8_bf16rope":
        cc = got.shape[-1]
        assert_within_ulp(got[..., : cc - 64], want[..., : cc - 64], "fp8", n_ulp, sl[..., : cc - 64],
                          what=what + "[fp8 dims]")
        assert_within_ulp(got[..., cc - 64:], want[..., cc - 64:], "bf16", n_ulp, sl[..., cc - 64:],
                          what=what + "[bf16 dims]")
        return
    if fmt == "f32":
        err = np.abs(got - want)
        assert err.max() <= 1e-5, f"{what}: f32 max error {err.max():.3g}"
        return
    tol = n_ulp * np.maximum(ulp_of(want, fmt), ulp_of(got, fmt)) + sl + 1e-300
    bad = np.abs(got - want) > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} values beyond {n_ulp} ulp; "
                           f"worst {np.abs(got - want).max():.3g}")


def certified(scores_oracle, bound, vis, k):
    """True if the row's selection cannot change under score errors <= bound.

    The k-th and (k+1)-th largest oracle scores must differ by more than twice
    the largest error bound of the row; rows with vis <= k are always certified.
    """
    if vis <= k:
        return True
    s = np.sort(scores_oracle[:vis])[::-1]
    return (s[k - 1] - s[k]) > 2 * bound[:vis].max()


def check_selection(idx_gpu, scores_gpu, scores_oracle, bound, vis, k, what=""):
    """Selection parity of one row.

    1. The GPU's selection equals the oracle's stable selection on the GPU's own
       fp32 scores (bit-exact select stage).
    2. Scores agree within the fp32 evaluation bound.
    3. On a certified row the GPU selection equals the oracle's; otherwise every
       entry clearly above the k-th score is selected and none clearly below.
    Returns True when the row was certified."""
    sg = np.asarray(scores_gpu[:vis], np.float64)
    so = np.asarray(scores_oracle[:vis], np.float64)
    want_sel = O.topk(sg[None], [vis], k)[0]
    assert np.array_equal(idx_gpu, want_sel), f"{what}: select stage differs from the oracle's select"
    err = np.abs(sg - so)
    assert np.all(err <= bound[:vis] + 1e-30), f"{what}: score error {err.max():.3g} > bound"
    osel = O.topk(so[None], [vis], k)[0]
    if certified(so, bound, vis, k):
        assert np.array_equal(idx_gpu, osel), f"{what}: certified row selects differently"
        return True
    kth = np.sort(so)[::-1][k - 1]
    kp1 = np.sort(so)[::-1][k]
    mb = 2 * bound[:vis].max()
    chosen = set(int(i) for i in idx_gpu if i >= 0)
    assert all(i in chosen for i in np.nonzero(so > kth + mb)[0]), f"{what}: missed a clear winner"
    assert not any(so[i] < kp1 - mb for i in chosen), f"{what}: picked a clear loser"
    return False
