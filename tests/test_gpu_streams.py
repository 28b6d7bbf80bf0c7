"""Calls made at once from several host threads, each on a HIP stream of its own.

The library keeps no state between calls and enqueues every launch on the caller's stream, so
concurrent calls on different streams may run side by side on the GPU and must each give what
the oracle gives for that call's own inputs.  Each thread repeats both operations on fresh
copies of its inputs; every copy is compared with the oracle (the first element by element
through the parity helpers, the others bit for bit against the first).
"""
import threading

import pytest
import torch

import rope_partial_inplace_amd as ra
import rope_workloads as W
from parity import check_bits_equal
from test_gpu_parity import DEV, check_inplace, compare_cache_case

pytestmark = pytest.mark.gpu

THREADS, REPEATS = 4, 6


def make_cases(i):
    inp = W.inplace_case(f"threads_inplace_{i}", 2, 64, 4, 96, torch.bfloat16, torch.float32,
                         [32, 96], seed=2000 + i, device=DEV, rotary_mode=i % 2)
    cc = W.cache_case(f"threads_cache_{i}", 300 + 17 * i, 8, 2, 128, 128 if i % 2 else 64,
                      torch.bfloat16, i % 2 == 0, 1024, seed=2100 + i, device=DEV)
    return inp, cc


def test_threads_each_on_its_own_stream():
    cases = [make_cases(i) for i in range(THREADS)]
    torch.cuda.synchronize()
    results = [None] * THREADS
    errors = []

    def work(i):
        try:
            inp, cc = cases[i]
            s = torch.cuda.Stream()
            xs, outs = [], []
            with torch.cuda.stream(s):
                for _ in range(REPEATS):
                    x = inp.x.clone()
                    ra.rope_partial_inplace(x, inp.cos, inp.sin, inp.rotary_mode,
                                            inp.partial_slice, stream=s)
                    qo, ko = torch.empty_like(cc.query), torch.empty_like(cc.key)
                    ra.rope_with_cos_sin_cache(cc.positions, cc.query, cc.key, cc.cache, None,
                                               cc.head_size, cc.is_neox, qo, ko, stream=s)
                    xs.append(x)
                    outs.append((qo, ko))
            s.synchronize()
            results[i] = (xs, outs)
        except Exception as e:  # reported from the main thread
            errors.append((i, repr(e)))

    workers = [threading.Thread(target=work, args=(i,)) for i in range(THREADS)]
    for w in workers:
        w.start()
    for w in workers:
        w.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (inp, cc) in enumerate(cases):
        xs, outs = results[i]
        check_inplace(inp.x.cpu(), xs[0], inp.cos, inp.sin, inp.partial_slice, inp.name,
                      inp.rotary_mode)
        compare_cache_case(cc, *outs[0])
        for r in range(1, REPEATS):
            check_bits_equal(xs[r].cpu(), xs[0].cpu(), f"{inp.name} repeat {r}")
            check_bits_equal(outs[r][0].cpu(), outs[0][0].cpu(), f"{cc.name} q repeat {r}")
            check_bits_equal(outs[r][1].cpu(), outs[0][1].cpu(), f"{cc.name} k repeat {r}")
