"""Block selection with a second-order block statistic (test infrastructure only).

The abstract on the page "CoSA: Accelerating Long-Context Inference via
Proxy-Kernel Co-Designed Sparse Attention" presents COBS (Cumulant Order Block
Sparse attention): block selection reduces to ranking blocks by attention mass
(the sum of a block's attention scores); a cumulant expansion shows that
scoring a block through a compact summary of its keys is a first-order
approximation of that mass; COBS stores a compressed second-order statistic
per block in addition. The pages give no formula. PARITY UNPINNED by the pages
for every choice below; the functions are pinned only against the mathematics
of the expansion (closed forms, limits) and against the first-order block path.

Reading:
  * for a query q and a block B of n_B visible keys k_t, the mass is
    M_B = sum_t exp(q . k_t) = n_B E_t[exp(X)] with X = q . k_t, and
    log E[exp(X)] = k1 + k2 / 2 + k3 / 6 + ... with cumulants k1 = q . mu_B and
    k2 = q^T Sigma_B q (mu_B, Sigma_B: mean and covariance of the block's keys);
  * first order: log M_B ~ log n_B + q . mu_B, a score of the block's mean key
    (the Eq. 2 mean pooling of the SparDA summary page, over the whole block);
  * second order, with the diagonal of Sigma_B as the compressed statistic:
    log M_B ~ log n_B + q . mu_B + 1/2 sum_c q_c^2 var_{B,c};
  * statistics exist for complete 64-token blocks only (candidate blocks are
    complete whenever at least one local block is kept), so log n_B = log 64 is
    a common constant and is left out of the score;
  * mu and var are the plain fp64 mean and population variance (mean of the
    squared deviations from the fp64 mean) of each channel over the block's 64
    keys, each rounded once, to nearest with ties to even, to the key dtype
    (numerics.round_once). The fp64 arithmetic is exact for the mean of 64 bf16
    or fp32 keys of ordinary range and within about 2^-46 relative for the
    variance, far below one unit in the last place of either key dtype, so an
    implementation that rounds an fp64 (or exact) result once agrees to 1 ulp;
  * a group's block score is the Eq. 6 form over the estimated log-masses
    (sum over the group's heads of each head's softmax over the blocks), or,
    in raw-sum mode (one Forecast vector, "Compact Forecast Indexer"), the sum
    of the estimates; top-k and the Eq. 1 union as in oracle.select.
Arithmetic fp64 from the statistics on.
"""
import numpy as np

from .numerics import round_once
from .select import SOFTMAX_SUM, RAW_SUM, candidate_sets, top_k_blocks, SelectParams
from .compress import n_blocks

BLOCK = 64


def block_stats(K: np.ndarray, L: int, dtype: str):
    """(mu, var) [L // 64, d] of the complete blocks of K[:L]: fp64 mean and
    population variance per channel, each rounded once to dtype ("f32" or
    "bf16")."""
    nbc = L // BLOCK
    d = K.shape[1]
    rows = np.asarray(K[:nbc * BLOCK], dtype=np.float64).reshape(nbc, BLOCK, d)
    mu = rows.mean(axis=1)
    var = ((rows - mu[:, None, :]) ** 2).mean(axis=1)
    return round_once(mu, dtype), round_once(var, dtype)


def cobs_log_mass(sel: np.ndarray, mu: np.ndarray, var: np.ndarray, order: int = 2) -> np.ndarray:
    """Estimated log-mass minus log 64 of every block with statistics, per
    selector head: [G, nbc] fp64 (order 1: q . mu; order 2: + 1/2 q^2 . var)."""
    q = np.asarray(sel, dtype=np.float64)
    est = q @ np.asarray(mu, dtype=np.float64).T
    if order == 2:
        est = est + 0.5 * (q * q) @ np.asarray(var, dtype=np.float64).T
    elif order != 1:
        raise ValueError(order)
    return est


def cobs_block_scores(sel, mu, var, nb: int, mode: str, order: int = 2) -> np.ndarray:
    """Group score of each of nb visible blocks (-inf for blocks without statistics)."""
    out = np.full(nb, -np.inf)
    nbc = min(mu.shape[0], nb)
    if nbc == 0:
        return out
    est = cobs_log_mass(sel, mu[:nbc], var[:nbc], order)         # [G, nbc]
    if mode == RAW_SUM:
        out[:nbc] = est.sum(axis=0)
    elif mode == SOFTMAX_SUM:
        m = est.max(axis=1, keepdims=True)
        e = np.exp(est - m)
        out[:nbc] = (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
    else:
        raise ValueError(mode)
    return out


def select_blocks_cobs(sel, mu, var, L: int, p: SelectParams, order: int = 2,
                       return_scores: bool = False):
    """Eq. 1 union of init, local and the top-k blocks by the COBS score."""
    nb = n_blocks(L)
    nbc = L // BLOCK
    BS = cobs_block_scores(sel, mu[:nbc], var[:nbc], nb, p.score_mode, order)
    init, local, cand = candidate_sets(nb, p.n_init, p.n_local)
    blocks = sorted(set(init) | set(local) | set(top_k_blocks(BS, cand, p.top_k)))
    return (blocks, BS) if return_scores else blocks
