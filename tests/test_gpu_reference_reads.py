"""The benchmarks' read-only reference kernels (pkv_stream_read, pkv_gather_read) reach
every byte they are given, in every load shape.

Both kernels fold every 32-bit word they load into one word per thread and store it to
`sink` only when it equals 0x5EED5EED.  With pools of zeros and that value planted in one
word, the sink is written exactly when the read loaded that word: planted at the end of
the last piece of the list (or of the buffer), it is written; planted in a piece the
list leaves out, it is not.  The piece list is a permutation of distinct pieces, so no
thread loads the planted word twice (which would cancel it).
"""

import numpy as np
import pytest
import torch

from paged_attention_decode_kv_amd import binding

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
MARK = 0x5EED5EED


def _as_i32(x: int) -> int:
    return x - (1 << 32) if x >= (1 << 31) else x


def _pools(piece_bytes: int, n_slots: int):
    words = piece_bytes * n_slots // 4
    k = torch.zeros(words, dtype=torch.int32, device=DEV)
    v = torch.zeros(words, dtype=torch.int32, device=DEV)
    return k, v


def _gather_sink(k, v, offsets, piece_bytes, gpc, waves, ppw):
    pieces = binding.GatherPieces(k, v, offsets, piece_bytes)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    binding.gather_read(pieces, sink, gpc, waves, ppw)
    torch.cuda.synchronize()
    return int(sink.item())


@pytest.mark.parametrize("waves,ppw", binding.GATHER_SHAPES)
@pytest.mark.parametrize("piece_bytes", [64, 256, 4096 + 256])
def test_gather_read_reaches_the_last_piece(waves, ppw, piece_bytes):
    # 2.5 passes of the largest grid used here (CUs x 3 workgroups x 8 waves x 4 loads,
    # each load a whole piece of 4352 bytes or 1024 / piece_bytes pieces of 64 and 256),
    # plus a count no shape divides; 4352-byte pieces leave a second 4 KB step with 16 of
    # 64 lanes live, and pieces of at most 1 KB are read by lane groups
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    per = 1024 // piece_bytes if piece_bytes <= 1024 else 1
    n = cus * 3 * 8 * 4 * per * 5 // 2 + 7
    n_slots = n + 1000
    rng = np.random.default_rng(piece_bytes * 16 + waves * 4 + ppw)
    order = rng.permutation(n_slots)
    listed = order[:n].astype(np.int64) * piece_bytes
    left_out = int(order[n]) * piece_bytes
    k, v = _pools(piece_bytes, n_slots)
    last_word = (int(listed[-1]) + piece_bytes) // 4 - 1
    for gpc in (1, 3):
        for pool in (k, v):
            pool.view(-1)[last_word] = _as_i32(MARK)
            got = _gather_sink(k, v, listed, piece_bytes, gpc, waves, ppw)
            pool.view(-1)[last_word] = 0
            assert got == _as_i32(MARK), (gpc, "k" if pool is k else "v")
        # the first word of the first piece
        first_word = int(listed[0]) // 4
        v.view(-1)[first_word] = _as_i32(MARK)
        assert _gather_sink(k, v, listed, piece_bytes, gpc, waves, ppw) == _as_i32(MARK)
        v.view(-1)[first_word] = 0
        # a piece the list leaves out is not read
        k.view(-1)[left_out // 4 + 5] = _as_i32(MARK)
        assert _gather_sink(k, v, listed, piece_bytes, gpc, waves, ppw) == 0
        k.view(-1)[left_out // 4 + 5] = 0


def test_gather_read_refuses_other_shapes():
    k, v = _pools(256, 8)
    pieces = binding.GatherPieces(k, v, np.arange(4, dtype=np.int64) * 256, 256)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for waves, ppw in ((2, 2), (16, 1), (4, 3), (8, 8)):
        with pytest.raises(binding.PagedKVError, match="SHAPE"):
            binding.gather_read(pieces, sink, 1, waves, ppw)
    with pytest.raises(binding.PagedKVError, match="SHAPE"):
        binding.gather_read(pieces, sink, 17, 4, 2)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


@pytest.mark.parametrize("gpc", [1, 2, 3, 8])
def test_stream_read_reaches_the_last_word(gpc):
    # a length that is no multiple of the 32 KB runs
    words = (3 * 1024 * 1024 + 4096 + 16) // 4
    buf = torch.zeros(words, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for where in (words - 1, 0, words // 2 + 3):
        buf[where] = _as_i32(MARK)
        sink.zero_()
        binding.stream_read(buf, sink, gpc)
        torch.cuda.synchronize()
        buf[where] = 0
        assert int(sink.item()) == _as_i32(MARK), where
