"""Seeded synthetic inputs shared by the CPU oracle, the tests and the bench.

Only input generation lives here (layouts of packed samples and random
activations); no mask predicate, attention arithmetic or planning.
"""
from .layouts import (WINDOW_INF, Layout, config, CONFIGS, ring_toy, packed_text,
                      packed_multimodal, sliding_window, long_mixed, random_small, video_group,
                      permuted)
from .tensors import toy_qkv, randn_bf16, qkv

__all__ = ["WINDOW_INF", "Layout", "config", "CONFIGS", "ring_toy", "packed_text",
           "packed_multimodal", "sliding_window", "long_mixed", "random_small", "video_group", "permuted",
           "toy_qkv", "randn_bf16", "qkv"]
