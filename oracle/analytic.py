"""Closed forms the pages print around the tensor-parallel sublayer.

TEST INFRASTRUCTURE ONLY.  Exact rational arithmetic (fractions.Fraction)
for the pipeline bubble, and integer byte counts for the all-reduce volumes.
They are pinned by tests against the values the pages print.
"""
from __future__ import annotations

from fractions import Fraction


def bubble_fraction(stages: int, micro_batches: int) -> Fraction:
    """Idle fraction of the whole step, (K-1)/(M+K-1).

    "Tensor and Pipeline Parallelism" (roadtointelligence), section
    "Pipeline parallelism: an assembly line"; "7.9 Tensor and pipeline
    parallelism" section 3.2 (P_p stages, M micro-batches); "Parallelism II:
    model", "Pipeline parallelism" (the m+p-1 slot form).
    """
    if stages < 1 or micro_batches < 1:
        raise ValueError("need at least one stage and one micro-batch")
    return Fraction(stages - 1, micro_batches + stages - 1)


def bubble_vs_useful(stages: int, micro_batches: int) -> Fraction:
    """Idle time relative to the useful work, (p-1)/m ("Parallelism II: model")."""
    if stages < 1 or micro_batches < 1:
        raise ValueError("need at least one stage and one micro-batch")
    return Fraction(stages - 1, micro_batches)


def bubble_interleaved_step(stages: int, micro_batches: int, v: int) -> Fraction:
    """Interleaved schedule, whole-step form: (1/v) (P-1)/(M+P-1) ("7.9 ..." section 3.4)."""
    return bubble_fraction(stages, micro_batches) / v


def bubble_interleaved_useful(stages: int, micro_batches: int, v: int) -> Fraction:
    """Interleaved schedule, useful-work form: (p-1)/(v m) ("Parallelism II: model")."""
    return bubble_vs_useful(stages, micro_batches) / v


def allreduce_payload_elems(batch: int, seq: int, d: int) -> int:
    """Elements in one TP all-reduce of the activations: B*T*d ("7.9 ..." section 2.1 box)."""
    return batch * seq * d


def ring_allreduce_bytes_per_gpu(n_gpus: int, payload_bytes: int) -> Fraction:
    """A ring all-reduce moves 2(N-1)/N times the payload per GPU (S17, "Mechanics")."""
    return Fraction(2 * (n_gpus - 1), n_gpus) * payload_bytes


def tp_decode_comm_bytes_per_step(layers: int, batch: int, d: int, n_gpus: int,
                                  bytes_per_elem: int = 2) -> Fraction:
    """Per-GPU all-reduce bytes per decode step: two all-reduces of batch x d per layer.

    S17 "Mechanics": the payload is batch x d_model x 2 bytes; two
    all-reduces per layer.
    """
    payload = batch * d * bytes_per_elem
    return 2 * layers * ring_allreduce_bytes_per_gpu(n_gpus, payload)


def allreduces_per_forward(layers: int) -> int:
    """Two all-reduces (attention, FFN) per block in the forward pass ("7.9 ..." section 2.2)."""
    return 2 * layers


def weight_bytes_per_device(params: float, bytes_per_param: int, T_p: int) -> float:
    """Each matrix is sharded T_p ways, so a device holds 1/T_p of the weights ("7.9 ..." 2.3)."""
    return params * bytes_per_param / T_p


def gqa_tp_allowed(n_heads: int, n_kv_heads: int, T_p: int) -> bool:
    """T_p must divide both head counts (S17, "Attention shards by head, and GQA caps the degree")."""
    return n_heads % T_p == 0 and n_kv_heads % T_p == 0


def layout_devices(*degrees: int) -> int:
    """Devices used by a composed layout: the product of the per-axis degrees."""
    out = 1
    for g in degrees:
        out *= g
    return out
