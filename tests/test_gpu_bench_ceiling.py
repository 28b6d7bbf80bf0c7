"""The measurement kernels of bench_ceiling.hip do the work their timings stand for.

bench.py divides each RoPE kernel's time by one of these kernels' time on the same bytes, so a
ceiling kernel that skipped part of its copy would flatter nothing but would make the ratio
meaningless.  Each test runs one entry point on seeded bytes and checks every byte it was meant
to write (and that the bytes around stay as they were): the dense copy at sizes that leave a
ragged last workgroup, the NeoX pair-unit copy with a ragged last wavefront, and the in-place
row pattern, which must leave x exactly as it found it.
"""
import os

import pytest
import torch

import bench

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not os.path.exists(bench.CEILING_LIB),
                                 reason="libbench_ceiling.so not built")]

DEV = torch.device("cuda:0")
GUARD = 4096  # bytes past the end of each output that must stay untouched


def random_bytes(n, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV, generator=g)


def stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("nbytes", [16, 16 * 63, 16 * 64, 16 * 1_000_003, 64 << 20])
def test_dense_copy_writes_every_byte(nbytes):
    lib = bench.load_ceiling()
    src = random_bytes(nbytes, seed=nbytes % 9973)
    dst = torch.full((nbytes + GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
    assert lib.ceiling_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())


@pytest.mark.parametrize("heads,head_bytes,rows_per_lane", [
    (1001, 256, 1), (1001, 256, 2),   # 8 lanes a head, 8 heads a wavefront: ragged last wave
    (77, 64, 2),                      # 2 lanes a head, 32 heads a wavefront
    (5, 2048, 2),                     # a whole wavefront per head
    (3, 96, 1),                       # 3 lanes a head, 21 heads a wavefront: lane 63 idle
])
def test_pair_unit_copy_writes_every_head(heads, head_bytes, rows_per_lane):
    lib = bench.load_ceiling()
    n = heads * head_bytes
    src = random_bytes(n, seed=heads * 7 + head_bytes)
    dst = torch.full((n + GUARD,), 0x5A, dtype=torch.uint8, device=DEV)
    assert lib.ceiling_pairs(dst.data_ptr(), src.data_ptr(), heads, head_bytes, rows_per_lane,
                             stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert bool((dst[n:] == 0x5A).all())


@pytest.mark.parametrize("rows,row_bytes,off,length,lane,rpl,side,rps,side_stream", [
    (8 * 4096, 1152, 1024, 128, 8, 1, 256, 1, True),    # [8,4096,1,576] slice [512,576) bf16
    (4 * 512 * 32, 384, 256, 128, 8, 4, 256, 32, False),  # heads sharing one cos/sin row
    (2 * 40_000, 256, 0, 256, 16, 2, 256, 2, True),      # dense f32 rows, two heads a row
    (1000, 96, 32, 48, 16, 1, 0, 1, False),              # no side arrays
])
def test_row_pattern_leaves_x_unchanged(rows, row_bytes, off, length, lane, rpl, side, rps,
                                        side_stream):
    lib = bench.load_ceiling()
    x = random_bytes(rows * row_bytes + GUARD, seed=rows + row_bytes)
    before = x.clone()
    n_side = -(-rows // rps) * max(side, 16)
    sa, sb = random_bytes(n_side, seed=1), random_bytes(n_side, seed=2)
    st = lib.ceiling_rows(x.data_ptr(), rows, row_bytes, off, length, lane, rpl, sa.data_ptr(),
                          sb.data_ptr(), side, rps, int(side_stream), stream())
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(x, before)
