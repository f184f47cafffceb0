"""Working-set delta between consecutive agent steps.

KVMem paper, Sec. 4.4 ("retrieval-aware hierarchical reuse"): with W_{t-1}
and W_t the working sets of two consecutive steps, the transition splits into
retained R_t = W_{t-1} & W_t, incoming L_t = W_t - W_{t-1} and outgoing
E_t = W_{t-1} - W_t. With G_{t-1} the blocks still resident in the bounded
GPU page pool, only L_t^physical = W_t - G_{t-1} must be staged in; the GPU
hits W_t & G_{t-1} keep their pages (V untouched; K re-encoded only when the
compact position changed). The displayed set equations were lost; these are
the set identities the prose states.
"""
from __future__ import annotations


def working_set_delta(W_prev, W_t, G_prev) -> dict:
    W_prev, W_t, G_prev = set(W_prev), set(W_t), set(G_prev)
    return {
        "retained": W_prev & W_t,
        "incoming": W_t - W_prev,
        "outgoing": W_prev - W_t,
        "hits": W_t & G_prev,
        "physical_in": W_t - G_prev,
    }
