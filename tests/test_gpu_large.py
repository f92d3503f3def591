"""The largest sizes the boundary accepts, checked by construction.

Rows hold one finite logit each (the rest -inf, masked vocabulary), so every
decision is fixed by where the finite logits sit, at any size:

- a greedy row's argmax is its finite entry;
- a draft token on the target's finite entry, with the draft row the same
  one-hot row, has p(x) = q(x) = 1 and is accepted whatever the uniform;
- a draft token where the target row is -inf has p(x) = 0 and is rejected,
  and the residual max(0, p - q) is then the target row itself, so the drawn
  token is the target's finite entry;
- with every slot accepted, the bonus draw from the one-hot row K returns
  its finite entry.

Two calls: more than 2^31 logits in one call (64-bit element offsets), and V
at its limit (2^31 - 65537, element indices next to INT_MAX), with the
finite entries placed at row starts and ends, segment edges and the ragged
last segment.  The expected outputs come from the placements alone.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

V_LIMIT = 2 ** 31 - 65537


def _positions(V: int, n: int, rng) -> np.ndarray:
    fixed = [0, V - 1, 8191, 8192, V - 8, V - 9, (V // 8192) * 8192, V // 2]
    extra = rng.integers(0, V, size=max(0, n - len(fixed)))
    return np.array((fixed + list(extra))[:n], dtype=np.int64)


def _run(b: int, K: int, V: int, seed: int):
    import lossless_draft_verification_amd as L
    rng = np.random.default_rng(seed)
    greedy = np.arange(b) % 2 == 0
    # finite entries: target row i of sequence s at y[s, i]; draft row i at y[s, i],
    # except at the rejected slot j[s] (z[s], where the target row is -inf)
    y = _positions(V, b * (K + 1), rng).reshape(b, K + 1)
    rng.shuffle(y.reshape(-1))
    j = rng.integers(0, K + 1, size=b)                     # j == K: every slot accepted
    z = (y[np.arange(b), np.minimum(j, K - 1)] + 1 + rng.integers(0, V - 1, size=b)) % V
    z = np.where(z == y[np.arange(b), np.minimum(j, K - 1)], (z + 1) % V, z)

    ninf = float("-inf")
    tgt = torch.full((b, K + 1, V), ninf, dtype=torch.bfloat16, device="cuda")
    drf = torch.full((b, K, V), ninf, dtype=torch.bfloat16, device="cuda")
    x = np.empty((b, K), np.int32)
    for s in range(b):
        for i in range(K + 1):
            tgt[s, i, int(y[s, i])] = 3.0
        for i in range(K):
            col = int(z[s]) if (not greedy[s] and i == j[s]) else int(y[s, i])
            drf[s, i, col] = 1.5
            x[s, i] = col
        if greedy[s] and j[s] < K:                         # greedy: a mismatching token at slot j
            x[s, j[s]] = int(z[s])
    temps = torch.from_numpy(np.where(greedy, 0.0, 0.8)).cuda()
    seeds = torch.from_numpy(np.arange(b, dtype=np.int64) + seed).cuda()
    r = L.mixed_accept(tgt, drf, torch.from_numpy(x).cuda(), temps, seeds)
    torch.cuda.synchronize()
    got = {f: getattr(r, f).cpu().numpy() for f in ("n_accepted", "tokens", "p_draft", "q_draft", "argmax")}
    del tgt, drf
    torch.cuda.empty_cache()

    for s in range(b):
        n = int(j[s])
        assert got["n_accepted"][s] == n, (s, got["n_accepted"][s], n)
        want_tok = [int(x[s, i]) for i in range(n)] + [int(y[s, n])] + [-1] * (K - n)
        np.testing.assert_array_equal(got["tokens"][s], want_tok, err_msg=f"sequence {s}")
        if greedy[s]:
            np.testing.assert_array_equal(got["argmax"][s], y[s], err_msg=f"argmax of sequence {s}")
            assert np.isnan(got["p_draft"][s]).all() and np.isnan(got["q_draft"][s]).all()
        else:
            assert (got["argmax"][s] == -1).all()
            for i in range(K):
                rejected = i == n
                assert got["p_draft"][s, i] == (0.0 if rejected else 1.0), (s, i, got["p_draft"][s, i])
                assert got["q_draft"][s, i] == 1.0, (s, i, got["q_draft"][s, i])


def test_more_than_2_31_logits_in_one_call():
    """b=4, K=8, V=2^26+37 (bf16): 2.4e9 target logits, 2.1e9 draft logits."""
    _run(4, 8, 2 ** 26 + 37, seed=101)


def test_vocabulary_at_its_limit():
    """b=2, K=1, V=2^31-65537 (bf16): 12.9 GB of logits."""
    _run(2, 1, V_LIMIT, seed=102)
