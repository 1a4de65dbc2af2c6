"""Seeded synthetic inputs shared by the oracle and the HIP path.

This package holds input generation only: rollout-DAG topologies (node and
mount tables) and seeded random tensors (for the gated-delta-rule layer the
query/key vectors are L2-normalised and the gates squashed into their ranges,
which is input preparation, not the layer's arithmetic).  It performs none of the method's
arithmetic -- no positions, no visibility, no attention -- so that the CPU
oracle and the GPU path can both consume it without sharing any computation.
"""
from .dags import DagSpec, DagBuilder, config1, config1_variant, config2, config3, config4, random_tiny_dag
from .tensors import bf16_round, normal, attn_inputs, gdn_inputs, logprob_inputs

__all__ = ["DagSpec", "DagBuilder", "config1", "config1_variant", "config2", "config3",
           "config4", "random_tiny_dag", "bf16_round", "normal", "attn_inputs", "gdn_inputs"]
