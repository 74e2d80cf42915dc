"""Rotation signs and JL matrices rebuilt from their seeds, each side with its own generator:
the GPU side through the library's host helpers (pq_make_signs, qjl_make_projection), the
oracle side through ``oracle.seeds``.  tests/test_oracle_seeds.py shows the two byte-equal on
the CPU, so both sides see the same D and G without either reading the other's output."""

import functools

from oracle import seeds


def gpu_signs(seed, d, device="cuda"):
    import kv_cache_quantization_amd as pq
    return pq.signs_tensor(seed, d, device)


def gpu_proj(seed, m, d, device="cuda"):
    import kv_cache_quantization_amd as pq
    return pq.projection_tensor(seed, m, d, device)


@functools.lru_cache(maxsize=64)
def _oracle_D(seed, d):
    return seeds.signs(seed, d)


@functools.lru_cache(maxsize=32)
def _oracle_G(seed, m, d):
    return seeds.projection_values(seed, m, d)


def oracle_D(seed, d):
    """+-1 float64 vector D of ``seed`` (oracle generator)."""
    return _oracle_D(int(seed), int(d)).copy()


def oracle_G(seed, m, d):
    """G of ``seed`` as float64 values [m, d] (oracle generator)."""
    return _oracle_G(int(seed), int(m), int(d)).copy()
