"""Oracle for the filter rules of Q-Filters -- TEST INFRASTRUCTURE.

All three estimators run in float64 with numpy's SVD as the library step and
return float64; callers round to float32 where the pages store float32 filters.

* ``compute_qfilters`` -- Q-Filters page, "Calibrated — the paper's actual
  mechanism": per query head, the top right singular vector v1 of the raw
  (not mean-centred) query matrix, signed by the sign of 1^T u1.
* ``average_gqa_filters`` -- same section: under grouped-query attention the
  filters of the query heads that share a KV head are averaged onto it; the
  pages state the result stays unit norm, read here as mean-then-renormalise.
  Query head h belongs to KV head h // (H_q / H_kv) (contiguous groups; the
  pages do not state the layout).
* ``estimate_filter_dir`` -- Q-Filters page, "Two filter sources" and
  "Key-SVD fallback": top right singular vector of the mean-centred first
  calib_tokens keys.  The pages call its sign ambiguous; after centring
  1^T u1 is identically zero, so the reading used here fixes the sign by making
  the entry of largest magnitude positive (lowest index on exact ties).  That
  sign rule is parity unpinned: the pages fix no sign for this source, so it is
  checked for self-consistency only (the direction itself is pinned).

Degenerate inputs (sigma_1 == sigma_2 up to 1e-12 relative, zero matrices,
a zero group mean, sgn(0)) follow the readings listed in the design notes:
errors for the first three, +1 for sgn(0).
"""
from __future__ import annotations

import numpy as np


class CalibError(ValueError):
    pass


def _top_right(x: np.ndarray):
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    if s.size == 0 or s[0] == 0.0:
        raise CalibError("zero matrix has no dominant direction")
    if s.size > 1 and s[0] - s[1] <= 1e-12 * s[0]:
        raise CalibError("top singular value is not separated (sigma1 == sigma2)")
    return u[:, 0], s, vt[0]


def qfilter_one_head(q: np.ndarray) -> np.ndarray:
    """Filter of one query head from its activations q [N, D] (no centring)."""
    q = np.asarray(q, dtype=np.float64)
    u1, _, v1 = _top_right(q)
    sgn = 1.0 if u1.sum() >= 0.0 else -1.0   # sgn(0) read as +1
    return sgn * v1


def compute_qfilters(acts: np.ndarray) -> np.ndarray:
    """acts [H_q, N, D] -> filters [H_q, D] (float64, unit norm)."""
    acts = np.asarray(acts, dtype=np.float64)
    return np.stack([qfilter_one_head(acts[h]) for h in range(acts.shape[0])])


def average_gqa_filters(filters: np.ndarray, n_kv_heads: int) -> np.ndarray:
    """filters [H_q, D] -> [n_kv_heads, D]: mean over each contiguous group, renormalised."""
    f = np.asarray(filters, dtype=np.float64)
    hq = f.shape[0]
    if n_kv_heads <= 0 or hq % n_kv_heads:
        raise CalibError("H_q must be a multiple of n_kv_heads")
    grp = hq // n_kv_heads
    out = np.empty((n_kv_heads, f.shape[1]))
    for j in range(n_kv_heads):
        m = f[j * grp:(j + 1) * grp].mean(axis=0)
        nrm = np.linalg.norm(m)
        if nrm == 0.0:
            raise CalibError("group mean is zero")
        out[j] = m / nrm
    return out


def estimate_filter_dir(keys: np.ndarray) -> np.ndarray:
    """Key-SVD fallback direction from keys [n, D] (float64, unit norm)."""
    x = np.asarray(keys, dtype=np.float64)
    x = x - x.mean(axis=0, keepdims=True)
    _, _, v1 = _top_right(x)
    i = int(np.argmax(np.abs(v1)))       # first index of the largest magnitude
    return v1 if v1[i] > 0 else -v1


def save_artifact(path: str, filters: np.ndarray, model_id: str, n_samples: int, dataset: str,
                  version: int = 1) -> None:
    """Write a calibration artifact (uncompressed .npz) with the fields the pages list."""
    np.savez(path, filters=np.asarray(filters, dtype=np.float32), model_id=np.array(model_id),
             version=np.array(version, dtype=np.int64), n_samples=np.array(n_samples, dtype=np.int64),
             dataset=np.array(dataset))
