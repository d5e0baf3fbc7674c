"""SICS block scores (oracle).

SPADE summary (gist.science/ja/paper/2608.03335), "The solution" part 2: instead of
guessing which blocks to keep, the scheme step splits the tokens into small groups
and checks how strongly the members of each group agree; a group that agrees is
important.  The score is the Sum of Intra-block Cosine Similarities.

Readings taken (the page gives the name and the idea, not a formula):
  * the sum runs over all ordered token pairs (i, j) of a block, i = j included;
  * a zero token row has no direction and contributes nothing;
  * the score is computed per (batch, head, block) for whichever token tensor the
    caller passes (the page does not say Q or K);
  * the selection rule that turns scores into kept blocks is not on the page and
    is not part of this function (parity unpinned for any such rule).
"""
import numpy as np


def block_sics(x, block):
    """x: [B, N, H, D] -> scores [B, H, ceil(N / block)] (fp64), by the definition
    sum_{i, j in block} cos(x_i, x_j), evaluated pair by pair (a Gram matrix)."""
    x = np.asarray(x, dtype=np.float64)
    B, N, H, _ = x.shape
    nb = -(-N // block)
    out = np.zeros((B, H, nb))
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                rows = x[b, i * block:min(N, (i + 1) * block), h]
                norm = np.linalg.norm(rows, axis=1)
                unit = np.divide(rows, norm[:, None], out=np.zeros_like(rows), where=norm[:, None] > 0)
                out[b, h, i] = (unit @ unit.T).sum()
    return out
