"""Print the quantiser-variant diagnostics (score KL, output error) as a
markdown table.  Test infrastructure: calls only the oracle and the seeded
input generators.

    python -m oracle.variant_report
"""
from __future__ import annotations

import numpy as np

from bit_rotated_kv_int2_amd import synth

from . import oscar_ref as R
from . import variants as V

D = 128


def workload_errors(name: str, n_tokens: int = 2048, n_cal: int = 512, n_heads: int | None = None):
    """Mean (score KL, output error) per variant over the KV heads of layer 0.
    Queries: the decode queries and 60 calibration queries of every query
    head of the KV head; every one of the first n_tokens tokens quantised."""
    wl = synth.WORKLOADS[name]
    q, k, v = synth.calibration_set(wl, 0, n_cal=n_cal)
    qf, kf, vf = (synth.bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v))
    kb, vb = synth.kv_tokens(wl, 0, 0, 0, n_tokens)
    qd = synth.bf16_bits_to_f32(synth.decode_queries(wl, 0)[0]).astype(np.float64)
    G = wl.n_q // wl.n_kv
    acc = {kind: [] for kind in V.KINDS}
    for h in range(n_heads or wl.n_kv):
        cal = R.calibrate_head(qf[h * G:(h + 1) * G], kf[h], vf[h], 1 / np.sqrt(D))
        kt = synth.bf16_bits_to_f32(kb[:, h]).astype(np.float64)
        vt = synth.bf16_bits_to_f32(vb[:, h]).astype(np.float64)
        qs = np.concatenate([qd[h * G:(h + 1) * G], qf[h * G:(h + 1) * G, :60].reshape(-1, D)])
        for kind in V.KINDS:
            acc[kind].append(V.attention_errors(qs, kt, vt, V.variant_calibration(kind, cal, kf[h], vf[h]),
                                                1 / np.sqrt(D)))
    return {kind: tuple(np.mean(np.array(e), axis=0)) for kind, e in acc.items()}


def main():
    rows = [("tiny-4k (4 outlier channels x20)", workload_errors("tiny-4k")),
            ("qwen3-8b-32k-b1 layer 0, 8 KV heads (10 outlier pairs x20)", workload_errors("qwen3-8b-32k-b1"))]
    print("| workload | measure | naive INT2 | clip only | Hadamard only | OSCAR |")
    print("|---|---|---|---|---|---|")
    for name, e in rows:
        print(f"| {name} | score KL (nats) | " + " | ".join(f"{e[k][0]:.3f}" for k in V.KINDS) + " |")
        print(f"| {name} | output error | " + " | ".join(f"{e[k][1]:.3f}" for k in V.KINDS) + " |")


if __name__ == "__main__":
    main()
