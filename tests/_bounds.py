"""Error bounds shared by the GPU tests (no GPU needed to import)."""
import numpy as np


def cancel_bound(ins, o_ref, scale, drop, oracle_mod):
    """Bounds on the Frobenius norms of dQ and dK when the exact ones vanish.

    dS_ij = P_ij (s_d M_ij dP_ij - D_i) is formed from dP_ij (fp32 sums of
    16-bit products) and D_i = dO_i . O_i, which the kernels take from the
    stored 16-bit O (relative rounding 2^-8 for bf16).  So |dS_ij| <= P_ij E_i
    with E_i = 2^-7 |dO_i| (|O_i| + s_d max_j |V_j|), a factor 2 above the O
    rounding to cover the fp32 terms; with sum_j P_ij <= 1,
    |dQ_i| <= scale max|K| E_i and ||dK|| <= scale max|Q| sum_i E_i."""
    rn = lambda x: np.linalg.norm(x.reshape(-1, x.shape[-1]), axis=1)
    sd = 256.0 / oracle_mod.dropout_threshold(drop) if drop > 0 else 1.0
    e = 2.0 ** -7 * rn(ins["do"]) * (rn(o_ref) + sd * rn(ins["v"]).max())
    return dict(dq=scale * rn(ins["k"]).max() * float(np.linalg.norm(e)),
                dk=scale * rn(ins["q"]).max() * float(e.sum()))
