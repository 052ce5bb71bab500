"""Comparators that apply the GPU-vs-oracle tolerances.

* page ids: per (sequence, kv head) the GPU set may differ from the oracle's
  only in pages whose oracle score lies within `tie` of the oracle's k-th best
  score;
* tokens / accepted lengths: bit-exact, except that a sequence is compared only
  up to its first decision that the oracle places within `window` of its
  threshold (|u - p/q| for accepts, distance of u*sum(w) to the chosen bin's
  edges over sum(w) for draws).
"""
import numpy as np


def check_pages(gpu_sel, gpu_nsel, ref_sel, ref_nsel, ref_scores, k, tie=1e-4):
    assert np.array_equal(gpu_nsel, ref_nsel), (gpu_nsel, ref_nsel)
    B, H, _ = ref_sel.shape
    for b in range(B):
        for h in range(H):
            g = [int(x) for x in gpu_sel[b, h] if x >= 0]
            assert g == sorted(g), ("not ascending", b, h, g)
            r = [int(x) for x in ref_sel[b, h] if x >= 0]
            assert len(g) == len(r), (b, h)
            if g == r:
                continue
            sc = ref_scores[(b, h)]
            assert sc is not None, (b, h)
            kth = np.sort(sc)[::-1][k - 1]
            for j in set(g) ^ set(r):
                assert abs(sc[j] - kth) <= tie, (b, h, j, sc[j], kth)


def check_tokens(gpu_out, gpu_n, ref_out, ref_n, decisions, window=1e-6):
    """Compare a round's tokens; returns the number of sequences compared in full.

    Decisions before the first one within `window` of its threshold are
    compared exactly. If that first close decision is the round's final draw,
    the accepted count and every accepted draft are still compared; if it is
    an accept test at slot i, tokens before slot i are compared.
    """
    full = 0
    for b in range(len(ref_n)):
        close = [d for d in decisions[b] if d[2] <= window]
        if not close:
            assert int(gpu_n[b]) == int(ref_n[b]), (b, gpu_n[b], ref_n[b])
            assert np.array_equal(gpu_out[b], ref_out[b]), (b, gpu_out[b], ref_out[b])
            full += 1
            continue
        slot, kind, _ = close[0]
        if kind == "draw":
            assert int(gpu_n[b]) == int(ref_n[b]), (b, gpu_n[b], ref_n[b])
        assert np.array_equal(gpu_out[b, :slot], ref_out[b, :slot]), b
    return full
