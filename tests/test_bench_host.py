"""CPU tests of the benchmark's host logic: the algorithmic bytes and flops its
roofline fractions divide by, recomputed here from the tensors the workloads
move (shapes and dtypes of the seeded inputs), and the --only selection."""
import importlib.util
import os

import pytest
import torch

from gated_delta_rule_chunkwise_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def nbytes(shape, dtype):
    n = 1
    for s in shape:
        n *= s
    return n * torch.empty((), dtype=dtype).element_size()


def test_long_context_bytes_are_the_tensors_moved(bench):
    """q, k, log alpha, v read and o written ([T, H, 128] bf16 each), beta read
    ([T, H] bf16) and h_T written ([1, H, 128, 128] fp32): 2,690,646,016 B."""
    T, H, d = 65536, 32, 128
    bf, f32 = torch.bfloat16, torch.float32
    tensors = 5 * nbytes((T, H, d), bf) + nbytes((T, H), bf) + nbytes((1, H, d, d), f32)
    assert tensors == 2_690_646_016
    assert bench.chunk_alg_bytes(T * H, H, d, d) == tensors


def test_long_context_flops(bench):
    """Per token-head at C = 64, d = 128 (triangles counted as triangles):
    A and P Gram blocks (C-1)/2 d + (C+1)/2 d multiply-adds, T C^2/6, U and W
    (C-1)/2 (d_k + d_v), the three state products 3 d_k d_v and P U (C+1)/2 d_v;
    two flops per multiply-add.  294.65 GFLOP for the long-context call."""
    C, d = 64, 128
    mac = (C - 1) / 2 * d + (C + 1) / 2 * d + C * C / 6 + (C - 1) / 2 * (2 * d) + 3 * d * d + (C + 1) / 2 * d
    th = 65536 * 32
    assert bench.chunk_alg_flops(th, d, d) == pytest.approx(2 * mac * th, rel=1e-12)
    assert 2 * mac * th / 1e9 == pytest.approx(294.6527, abs=1e-3)


def test_decode_bytes_are_the_tensors_moved(bench):
    """One decode step: the fp32 state read and written once, q, k, log alpha,
    v read and o written (bf16), beta read: 1,084,243,968 B for B = 256,
    H = 32, d = 128."""
    B, H, d = 256, 32, 128
    bf, f32 = torch.bfloat16, torch.float32
    tensors = 2 * nbytes((B, H, d, d), f32) + 5 * nbytes((B, H, d), bf) + nbytes((B, H), bf)
    assert tensors == 1_084_243_968
    assert bench.decode_alg_bytes(B, H, d, d) == tensors


def test_packed_batch_bytes_count_both_states(bench):
    """The packed 32-sequence workload reads h0 and writes h_T per (sequence,
    head); the benchmark counts both."""
    lengths = I.seq_lengths(I.C2)   # the same first draw as the workload's inputs
    T, H, N = sum(lengths), I.C2.H, len(lengths)
    assert N == 32 and T == 154217
    bf = torch.bfloat16
    tensors = (5 * nbytes((T, H, 128), bf) + nbytes((T, H), bf) + 2 * nbytes((N, H, 128, 128), torch.float32))
    assert bench.chunk_alg_bytes(T * H, N * H * 2, 128, 128) == tensors


def test_only_choices_cover_every_timed_workload(bench):
    for name in ("c3", "prologue", "gdn_gated", "gdn_deltanet", "decoupled", "strong", "c0", "c1", "c2",
                 "c1_fp32", "bwd", "bwd_prologue", "bwd_decoupled", "bwd_gdn", "bwd_c2", "decode"):
        assert name in bench.ONLY
