"""Selection quality: exact block attention mass and the recall of a block set.

TEST INFRASTRUCTURE ONLY (see the package header).

Page "CoSA: Accelerating Long-Context Inference via Proxy-Kernel Co-Designed
Sparse Attention" (abstract): block selection reduces to ranking blocks by their
attention mass, the sum of a block's attention probabilities, and selecting the
blocks of largest mass recovers dense quality. The SparDA page ("Training",
Eq. 7) partitions a distribution into the k selected blocks kept one by one and
a single rest bucket holding the remaining mass.

Here, for one query head at the decode position (visible length L): the dense
probabilities a_t = softmax_t(scale * q . k_t) over t < L, summed per 64-token
block; the recall of a block set B is the sum of its blocks' masses (1 minus the
rest bucket). fp64 throughout.
"""
import numpy as np

from .compress import n_blocks

BLOCK = 64


def block_mass(q: np.ndarray, K: np.ndarray, L: int, scale: float) -> np.ndarray:
    """Attention mass of every block b < nb(L) for one query head: [nb(L)] fp64."""
    L = int(L)
    if L <= 0:
        return np.zeros(0)
    z = scale * (K[:L].astype(np.float64) @ q.astype(np.float64))
    a = np.exp(z - z.max())
    a /= a.sum()
    nb = n_blocks(L)
    mass = np.zeros(nb)
    for b in range(nb):
        mass[b] = a[BLOCK * b:BLOCK * (b + 1)].sum()
    return mass


def recall(mass: np.ndarray, blocks) -> float:
    """Mass captured by a block set (the complement of the rest bucket)."""
    return float(sum(mass[b] for b in blocks))


def rest_bucket_distribution(mass: np.ndarray, blocks) -> np.ndarray:
    """Eq. 7's top-k partitioned distribution: the selected blocks' masses in
    the order given, then the rest bucket."""
    sel = [mass[b] for b in blocks]
    return np.array(sel + [1.0 - sum(sel)])


def mass_optimal_blocks(mass: np.ndarray, k: int, n_init: int, n_local: int):
    """The set of the same shape as the method's (init, local, and k candidates)
    with the largest recall: the k candidates of largest mass, ties to the lower
    id."""
    nb = len(mass)
    init = list(range(min(n_init, nb)))
    local = list(range(max(0, nb - n_local), nb))
    cand = [b for b in range(nb) if b not in init and b not in local]
    top = sorted(cand, key=lambda b: (-mass[b], b))[:max(0, k)]
    return sorted(set(init) | set(local) | set(top))
