"""Second, independent derivation of the position terms: Appendix B of Dai et al.

Appendix B ("Efficient Computation of the Attention with Relative Positional
Embedding") collects term (b) of every (i, j) into an L x (M+L) matrix B and
term (d) into D.  It stores the projected encodings in reversed order,
Q_k = W_kR R_{M+L-1-k}, forms B~ = q Q^T and d~ = Q v, and obtains row i of B
(and of D) by shifting row i of B~ (and d~) to the left, so that the last row
(i = L-1) is B~ itself and row 0 is shifted the most.  Entries shifted in from
the right are the zeros of the printed matrices, i.e. the masked keys.

Used only as a pin for the oracle (it never indexes a distance i-j directly).
"""
import numpy as np


def position_terms(q, vb, r_rows, M):
    """Terms (b) and (d) for one head via the shift formulation.

    q [L, d] queries; vb [d] position bias; r_rows [M+L, d] with r_rows[p] =
    W_kR R_p in natural order; M = memory length.  Returns (Bm, Dm), each
    [L, M+L], zero where the printed matrices are zero.
    """
    L = q.shape[0]
    T = M + L
    Q = r_rows[:T][::-1]              # Q_k = W_kR R_{M+L-1-k}
    Bt = q @ Q.T                      # B~ = q Q^T, [L, M+L]
    dt = Q @ vb                       # d~ = Q v, [M+L]
    Bm = np.zeros((L, T))
    Dm = np.zeros((L, T))
    for i in range(L):
        s = L - 1 - i                 # left shift of row i
        Bm[i, : T - s] = Bt[i, s:]
        Dm[i, : T - s] = dt[s:]
    return Bm, Dm


def scores(q, k, r, u, vb, M, scale):
    """Full score matrix of one head, [L, M+L], -inf where Appendix B's B is 0.

    Content terms (a)+(c) are one matrix product (q + u) k^T; the position
    terms come from position_terms().
    """
    L = q.shape[0]
    T = M + L
    Bm, Dm = position_terms(q, vb, r, M)
    A = scale * ((q + u[None, :]) @ k.T + Bm + Dm)
    visible = np.zeros((L, T), dtype=bool)
    for i in range(L):
        # the printed row i has M+i+1 leading entries before its zeros
        visible[i, : M + i + 1] = True
    return np.where(visible, A, -np.inf)
