"""The streaming read behind the bench's measured read bandwidth (gqa_read_bandwidth).

Each workgroup of the read leaves the sum of the 32-bit words it read; over
every workgroup that is the sum of the whole buffer (mod 2^32) exactly when
every word was read once. Checked on ragged sizes (a tail smaller than one
round of loads, a buffer smaller than the grid) and grid sizes from one
workgroup to the largest.
"""
import pytest
import torch

from gqa_kv_cache_decode_amd import api

pytestmark = pytest.mark.gpu

MOD = 1 << 32


def _expected(words: torch.Tensor) -> int:
    return int(words.to(torch.int64).sum().item()) % MOD


@pytest.mark.parametrize("nwords,wgs", [
    ((16 << 20) // 4 + 12, 256),   # 16 MiB and 48 bytes: a ragged tail in the last workgroup
    ((16 << 20) // 4 + 12, 1),
    ((16 << 20) // 4 + 12, 7),
    (4, 2048),                     # one 16-byte chunk, most workgroups read nothing
    (4 * 1000, 2048),
    ((256 << 20) // 4, 256),       # the size the bench reads per launch, in parts
])
def test_read_bandwidth_reads_every_word_once(gpu_lib, nwords, wgs):
    g = torch.Generator(device="cuda").manual_seed(nwords + wgs)
    src = torch.randint(-(1 << 31), (1 << 31) - 1, (nwords,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.full((wgs,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    api.read_bandwidth(src, sink)
    torch.cuda.synchronize()
    got = int((sink.to(torch.int64) % MOD).sum().item()) % MOD
    assert got == _expected(src)


def test_read_bandwidth_rejects_a_ragged_byte_count(gpu_lib):
    src = torch.zeros(5, dtype=torch.int32, device="cuda")  # 20 bytes
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(Exception):
        api.read_bandwidth(src, sink)
