"""GPU tests of kda_chunk_fwd_noalloc, the chunk forward that allocates nothing:
its workspace is a scratch array the library holds on each device.  Each test
makes two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents), and checks them against kda_chunk_fwd on the same
inputs: to the bf16 bar (max-abs 5e-3, relative Frobenius 1e-2) where the two
entry points run different kernels, bitwise where they run the same one."""
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from kda_testutil import assert_close  # noqa: E402

from gated_delta_rule_chunkwise_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_chunkwise_amd as kda
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kda.load_library(kda.LIB_PATH)
    return kda


def _inputs(cfg, lengths, B):
    d = I.make_chunk_inputs(cfg, device=DEV, lengths=lengths)
    if B > 1:   # equal-length batch [B, T, H, d]
        T = lengths[0]
        for n in ("q", "k", "v", "log_alpha", "beta"):
            d[n] = d[n].reshape((B, T) + tuple(d[n].shape[1:])).contiguous()
    return d


def _both(kda, d, packed):
    """(o, h_T) of kda_chunk_fwd and of kda_chunk_fwd_noalloc on the same inputs."""
    cu = d["cu_seqlens"] if packed else None
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    o_ref, h_ref = kda.kda_chunk_fwd(*args, h0=d["h0"], cu_seqlens=cu)
    o = torch.full_like(o_ref, float("nan"))
    hT = torch.full_like(h_ref, float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    o2, h2 = kda.kda_chunk_fwd_noalloc(*args, h0=d["h0"], cu_seqlens=cu, o=o, h_T=hT)
    assert torch.cuda.memory_allocated() == before
    torch.cuda.synchronize()
    assert o2.data_ptr() == o.data_ptr() and h2 is hT
    return o_ref.cpu(), h_ref.cpu(), o2.cpu(), h2.cpu()


def test_noalloc_equal_length_matches_chunk_fwd(kda):
    """bf16 at d = 128, equal-length batches long enough to be cut into segments
    (the scratch holds the segment states): 1 x 4096 tokens at H = 4, then
    2 x 1000 tokens at H = 2."""
    for B, H, T, seed in ((1, 4, 4096, 51), (2, 2, 1000, 52)):
        cfg = I.ChunkConfig("noalloc", "bf16", "bf16", H=H, dk=128, dv=128, h0=True, gate="uniform", seed=seed)
        d = _inputs(cfg, [T] * B, B)
        o_ref, h_ref, o, h = _both(kda, d, packed=False)
        print("noalloc equal-length B=%d H=%d T=%d" % (B, H, T), flush=True)
        assert_close(o, o_ref, "bf16", "o B=%d T=%d" % (B, T))
        assert_close(h, h_ref, "bf16", "h_T B=%d T=%d" % (B, T))


def test_noalloc_packed_matches_chunk_fwd_bitwise(kda):
    """Packed batches run the fused kernel from both entry points: bitwise equal
    (the scratch holds the order of the sequences)."""
    for lens, seed in (([700, 64, 1, 1500, 333, 0, 129], 53), ([100, 65], 54)):
        cfg = I.ChunkConfig("noalloc", "bf16", "bf16", H=3, dk=128, dv=128, h0=True, seed=seed)
        d = _inputs(cfg, lens, 1)
        o_ref, h_ref, o, h = _both(kda, d, packed=True)
        print("noalloc packed lengths", lens, flush=True)
        assert torch.equal(o, o_ref)
        assert torch.equal(h, h_ref)


def test_noalloc_fp32_and_d64_match_chunk_fwd_bitwise(kda):
    """fp32 I/O (at d_k = 128 the chunkwise fp32 forward, its records, states
    and U in the scratch) and bf16 at d = 64 (the two-pass forward, its records
    in the scratch) run the kernels of kda_chunk_fwd: bitwise equal."""
    for io, dk, dv, lens, seed in (("f32", 128, 128, [300], 55), ("bf16", 64, 64, [2048, 2048], 56),
                                   ("bf16", 64, 128, [777], 57)):
        cfg = I.ChunkConfig("noalloc", io, io, H=2, dk=dk, dv=dv, h0=True, seed=seed)
        B = len(lens)
        d = _inputs(cfg, lens, B)
        o_ref, h_ref, o, h = _both(kda, d, packed=False)
        print("noalloc", io, dk, dv, lens, flush=True)
        assert torch.equal(o, o_ref)
        assert torch.equal(h, h_ref)


def test_noalloc_rejects_calls_beyond_its_scratch(kda):
    """A call whose workspace exceeds the scratch is refused before any launch."""
    cfg = I.ChunkConfig("noalloc", "bf16", "bf16", H=32, dk=64, dv=64, seed=58)
    d = _inputs(cfg, [8192] * 8, 8)
    o = torch.full((8, 8192, 32, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kda.KDAError) as ei:
        kda.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], o=o)
    assert ei.value.code == kda.KDA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
