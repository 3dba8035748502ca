"""The two 32-element block transforms and their inverses, float64, dense form.

The oracle always multiplies by the dense matrices (np.kron, scipy's Hadamard,
an explicit permutation gather); it never uses a factored or butterfly form.

* Kronecker (KroQuant page, §02): activations are cut into 32-element blocks and
  each block is multiplied by one invertible P = A (x) B, A 4x4 and B 8x8, acting on
  row vectors: y_blk = x_blk . kron(A, B).  One (A, B) pair per layer, shared by all
  blocks (the page's parameter-count claim only fits a shared pair).
* RPBH (OrbitQuant page, §03): X' = X.P.H.D with P a permutation, H block-Hadamard
  and D random signs.  Read literally: u = x.Pi with (x.Pi)_j = x_{pi(j)} over all K,
  then v = u . blockdiag(H32) with H32 the Sylvester Hadamard matrix, then
  y_j = v_j d_j / sqrt(32).  The 1/sqrt(32) makes R = Pi.blockdiag(H32).D/sqrt(32)
  orthogonal, as the page states R is.
* Dense block transform (KroQuant page, §01): the same per-block product with a full
  32x32 P, of which kron(A, B) is the factorized form.
* Per-block Kronecker factors (KroQuant page, §02, with one (A_b, B_b) pair per block
  index b instead of one per layer): y_blk_b = x_blk_b . kron(A_b, B_b).
* Offline fold (KroQuant §01; OrbitQuant §03): W' = P^-1 W (R^-1 = R^T), so that
  (XP)(P^-1 W) = XW.
"""

import numpy as np
import scipy.linalg

BLOCK = 32


def kron_block_matrix(A, B):
    """Dense 32x32 block transform kron(A, B) (A 4x4, B 8x8), float64."""
    A = np.asarray(A, dtype=np.float64).reshape(4, 4)
    B = np.asarray(B, dtype=np.float64).reshape(8, 8)
    return np.kron(A, B)


def apply_block_matrix(x, P32):
    """y = x . blockdiag(P32, ..., P32) for rows x [M, K] (K a multiple of 32)."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    blocks = x.reshape(M, K // BLOCK, BLOCK)
    return (blocks @ P32).reshape(M, K)


def kron_block_matrices(A, B):
    """Per-block dense transforms kron(A_b, B_b), [nb, 32, 32] float64, from A [nb, 4, 4]
    and B [nb, 8, 8]."""
    A = np.asarray(A, dtype=np.float64).reshape(-1, 4, 4)
    B = np.asarray(B, dtype=np.float64).reshape(-1, 8, 8)
    return np.stack([np.kron(a, b) for a, b in zip(A, B)])


def apply_block_matrices(x, Ps):
    """y_b = x_b . Ps[b] for every 32-block b of rows x [M, K], Ps [K/32, 32, 32]."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    blocks = x.reshape(M, K // BLOCK, BLOCK)
    return np.einsum("mbi,bij->mbj", blocks, np.asarray(Ps, dtype=np.float64)).reshape(M, K)


def hadamard32():
    """Sylvester-ordered 32x32 Hadamard matrix with +-1 entries (scipy's construction)."""
    return scipy.linalg.hadamard(BLOCK).astype(np.float64)


def rpbh_apply(x, perm, sign):
    """RPBH(x) = x . Pi . blockdiag(H32) . D / sqrt(32) for rows x [M, K]."""
    x = np.asarray(x, dtype=np.float64)
    perm = np.asarray(perm, dtype=np.int64)
    d = np.asarray(sign, dtype=np.float64)
    u = x[:, perm]                                   # (x.Pi)_j = x_{pi(j)}
    v = apply_block_matrix(u, hadamard32())
    return v * d / np.sqrt(32.0)


def rpbh_dense(perm, sign):
    """Dense K x K matrix R = Pi . blockdiag(H32) . D / sqrt(32) (small K only)."""
    perm = np.asarray(perm, dtype=np.int64)
    K = perm.shape[0]
    Pi = np.zeros((K, K))
    Pi[perm, np.arange(K)] = 1.0                     # Pi[pi(j), j] = 1
    Hb = np.kron(np.eye(K // BLOCK), hadamard32())
    D = np.diag(np.asarray(sign, dtype=np.float64))
    return Pi @ Hb @ D / np.sqrt(32.0)


def fold_kron(W_out_in, A, B):
    """W' = P^-1 W for the Kronecker transform, W given as [N][K] (row n = column n of W).

    P^-1 is blockdiag(inv(kron(A, B))), the inverse computed by LAPACK on the dense
    32x32 block.  Returns W'^T as [N][K] float64.
    """
    Wt = np.asarray(W_out_in, dtype=np.float64)
    Pinv = np.linalg.inv(kron_block_matrix(A, B))
    # W' = blockdiag(Pinv) W  <=>  W'^T = W^T . blockdiag(Pinv)^T
    return apply_block_matrix(Wt, Pinv.T)


def fold_dense(W_out_in, P32):
    """W' = P^-1 W for a dense 32x32 block transform P, W given as [N][K]; returns W'^T as
    [N][K] float64 (P^-1 from LAPACK on the dense block)."""
    Wt = np.asarray(W_out_in, dtype=np.float64)
    Pinv = np.linalg.inv(np.asarray(P32, dtype=np.float64).reshape(BLOCK, BLOCK))
    return apply_block_matrix(Wt, Pinv.T)


def fold_kron_blocks(W_out_in, A, B):
    """W' = blockdiag_b(inv(kron(A_b, B_b))) W for per-block factors, W given as [N][K];
    returns W'^T as [N][K] float64 (each inverse from LAPACK on its dense 32x32 block)."""
    Wt = np.asarray(W_out_in, dtype=np.float64)
    Pinv = np.linalg.inv(kron_block_matrices(A, B))
    return apply_block_matrices(Wt, np.transpose(Pinv, (0, 2, 1)))


def fold_rpbh(W_out_in, perm, sign):
    """W' = R^T W for RPBH, W given as [N][K]; returns W'^T as [N][K] float64."""
    Wt = np.asarray(W_out_in, dtype=np.float64)
    # W'^T = W^T R, and W^T R is exactly RPBH applied to the rows of W^T.
    return rpbh_apply(Wt, perm, sign)
