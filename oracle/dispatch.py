"""Model of the per-step backend rule (TEST INFRASTRUCTURE).

paperlayer.ai summary §3 "Per-step dispatch" and Appendix B.4 "Per-Step
Dispatch Trace"; reading card "Key ideas": every decode step looks at the
realised batch, forms M_eff = B * n_q / n_kv, and takes the dense (batched
GEMM) prefix backend when M_eff reaches the saturation threshold M_sat, the
cascade backend otherwise.  The comparison is ">=" (ties go to dense).
"""

BACKEND_CASCADE = 1
BACKEND_DENSE = 2


def m_eff(batch: int, n_q: int, n_kv: int) -> int:
    if n_kv <= 0 or n_q % n_kv:
        raise ValueError("n_q must be a multiple of n_kv")
    return batch * (n_q // n_kv)


def choose_backend(batch: int, n_q: int, n_kv: int, m_sat: int) -> int:
    return BACKEND_DENSE if m_eff(batch, n_q, n_kv) >= m_sat else BACKEND_CASCADE
