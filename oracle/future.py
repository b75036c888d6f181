"""Oracle for future-query importance scores of cached keys (fp64, plain definitions).

TEST INFRASTRUCTURE (see `oracle/__init__.py`): importable only by tests, the smoke check and the
benchmark's CPU baseline.

Source: Future Forcing summary page ("Riepilogo Tecnico: Future Forcing", gist.science), section
"Componenti Algorithmiche", module 1 (future-aware KV-cache eviction): proxies of future queries are
built from historical statistics, each cached key is scored by its predicted attention weight under
those proxies, and the eviction score mixes that prediction with a historical score through a weight
lambda; implementation detail 3: the per-token importance is computed without forming the full
attention matrix Q K^T.

Readings of points the page leaves open (its Eq. 2 is not on the page):
  * the importance of key j in head h is the attention weight it receives from a proxy query,
    softmax over all scored keys of tau q~_i . k_j, averaged over the proxy queries i; so the
    importances of one head sum to 1;
  * a token's score is the mean of its importances over the heads (a token is evicted as a whole);
  * the hybrid score is lambda * future + (1 - lambda) * historical;
  * building the proxies (RoPE at future positions applied to the mean of the historical pre-RoPE
    queries) depends on the model's rotary layout, which the page does not give: proxies are inputs.
"""
from __future__ import annotations

import numpy as np


def importance(q_proxy, k, scale: float, block: int = 256) -> np.ndarray:
    """[H, n_k] mean over proxy queries of softmax_j(tau q~_i . k_j), per head, in float64.

    q_proxy: [n_p, H, d_h] (n_p >= 1), k: [n_k, H, d_h] (n_k >= 1)."""
    q = np.asarray(q_proxy, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n_p, H, _ = q.shape
    n_k = k.shape[0]
    out = np.zeros((H, n_k), dtype=np.float64)
    for h in range(H):
        for i0 in range(0, n_p, block):
            s = scale * (q[i0:i0 + block, h, :] @ k[:, h, :].T)     # [b, n_k]
            s -= s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[h] += (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
    return out / n_p


def token_scores(imp) -> np.ndarray:
    """Per-token score: mean of the per-head importances, [n_k]."""
    return np.asarray(imp, dtype=np.float64).mean(axis=0)


def hybrid(future, historical, lam: float) -> np.ndarray:
    """Eviction score lambda * future + (1 - lambda) * historical."""
    return lam * np.asarray(future, dtype=np.float64) + (1.0 - lam) * np.asarray(historical, dtype=np.float64)
