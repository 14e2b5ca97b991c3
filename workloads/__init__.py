"""Seeded synthetic verify workloads shared by the oracle tests, the GPU tests and the benchmark."""
from .synth import (BATCHED, BY_NUMBER, GREEDY, HEAVY, INTERACTIVE, MIXED, QWEN3_VOCAB, TINY,
                    WORKLOADS, FlatInputs, Inputs, Workload, bf16_bits_to_f32, flatten, generate,
                    markov_base, markov_factors, markov_sampling,
                    schedule_confidences, sweep_workload, to_bf16_bits)
