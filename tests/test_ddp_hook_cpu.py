"""The DDP communication hook's orchestration on CPUs, with two gloo ranks.

The hook runs four library calls and two collectives per bucket:
- the norm term, and an all-reduce of it;
- the norm from the combined term;
- the rank's codes in the word layout at worker index = rank;
- an integer SUM all-reduce of the words, then dequantization with n = world.

Here the four calls are stand-ins built from the CPU oracle (the library
needs a GPU), so the test checks what the hook itself decides: the combine
operation of the norm term, the worker index, the code width for `world`
workers, the n used to dequantize, and the per-(bucket, call) seeds. Every
bucket's mean on both ranks must equal, bit for bit, the oracle's mean over
the two ranks' buckets stacked as one [2, d] input and run in one process.
Both ranks' gradients must also agree after DDP writes them back.
"""
import ctypes
import math
import os
import socket
import tempfile
from types import SimpleNamespace

import numpy as np
import pytest

torch = pytest.importorskip("torch")
import torch.distributed as dist  # noqa: E402

import oracle  # noqa: E402

SCH = {"L": oracle.SCHEME_L, "E": oracle.SCHEME_E}
CASES = [("L", 7, 2.0, 2.0), ("E", 6, math.inf, 2.0), ("L", 127, 2.0, math.inf),
         ("E", 9, math.inf, math.inf)]


def oracle_ops():
    """The hook's four device calls, computed by the oracle on CPU tensors."""
    def norm_term(x, q, p, term=None, workspace=None):
        _, pw = oracle.global_norm(x.detach().numpy(), q, p)
        t = float(pw[0])  # sum of squares (q = 2) or max |x| (q = inf)
        if math.isinf(q) and not math.isinf(p):
            t = t * t      # the term of (inf, 2) is the square of the max (exact in fp64)
        return torch.tensor([t], dtype=torch.float64)

    def norm_from_term(term, q, p, norm=None):
        T = np.array([float(term[0])], dtype=np.float64)
        qq = math.inf if (math.isinf(q) and math.isinf(p)) else 2.0
        N = oracle.lib().oracle_norm_from_partials(T.ctypes.data_as(ctypes.c_void_p), 1, qq, qq)
        return torch.tensor([N], dtype=torch.float32)

    def quantize_words(x, s, scheme, norm, seed, W, worker_base=0, words=None):
        codes = oracle.quantize(x.detach().numpy(), float(norm[0]), s, SCH[scheme], seed,
                                worker_base=worker_base)
        rows = oracle.pack_words(codes, W, oracle.top_code(s, SCH[scheme]))
        return torch.from_numpy(rows.view(np.int32).copy())

    def dequantize_words(wsum, n, d, s, scheme, W, norm, mean=None):
        M = oracle.top_code(s, SCH[scheme])
        sums = oracle.unpack_word_sums(wsum.numpy().view(np.uint32), n, d, W, M)
        m = torch.from_numpy(oracle.dequantize(sums, n, float(norm[0]), s, SCH[scheme]))
        if mean is None:
            return m
        mean.copy_(m)
        return mean

    return SimpleNamespace(norm_term=norm_term, norm_from_term=norm_from_term,
                           quantize_words=quantize_words, dequantize_words=dequantize_words)


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _rank(rank, world, port, outdir):
    from torch.nn.parallel import DistributedDataParallel as DDP

    from allreduce_compatible_gradient_amd.ddp import GlobalQSGDState, global_qsgd_hook
    dist.init_process_group("gloo", init_method=f"tcp://127.0.0.1:{port}", rank=rank,
                            world_size=world)
    try:
        for c, (scheme, s, q, p) in enumerate(CASES):
            torch.manual_seed(0)  # the same initial weights on every rank
            model = torch.nn.Sequential(*[m for _ in range(4)
                                          for m in (torch.nn.Linear(64, 64), torch.nn.Tanh())])
            ddp = DDP(model, bucket_cap_mb=0.01)  # one bucket per layer or so after the first step
            state = GlobalQSGDState(scheme=scheme, s=s, q=q, p=p, seed=7 + c, ops=oracle_ops())
            seeds = []
            plain_next = state.next_seed

            def next_seed(i, plain_next=plain_next, seeds=seeds):
                sd = plain_next(i)
                seeds.append(sd)
                return sd
            state.next_seed = next_seed
            recs = []
            step = [0]

            def hook(st, bucket, recs=recs, seeds=seeds, step=step):
                inp = bucket.buffer().detach().clone()
                fut = global_qsgd_hook(st, bucket)
                sd, it, idx = seeds[-1], step[0], bucket.index()
                # completions may come back in another order on each rank: key by (step, bucket)
                return fut.then(lambda f: recs.append((it, idx, inp.numpy(),
                                                       f.value().detach().clone().numpy(), sd))
                                or f.value())
            ddp.register_comm_hook(state, hook)
            g = torch.Generator().manual_seed(100 + rank)
            for it in range(3):
                step[0] = it
                ddp.zero_grad()
                xin = torch.randn(16, 64, generator=g)
                ddp(xin).pow(2).sum().backward()
            recs.sort(key=lambda r: (r[0], r[1]))
            recs = [r[1:] for r in recs]
            grads = np.concatenate([prm.grad.detach().numpy().ravel() for prm in model.parameters()])
            np.savez(os.path.join(outdir, f"case{c}_rank{rank}.npz"), grads=grads,
                     idx=np.array([r[0] for r in recs]), seed=np.array([r[3] for r in recs],
                                                                       dtype=np.uint64),
                     **{f"in{k}": r[1] for k, r in enumerate(recs)},
                     **{f"out{k}": r[2] for k, r in enumerate(recs)})
            dist.barrier()
    finally:
        dist.destroy_process_group()


def test_two_ranks_reproduce_the_single_process_operator():
    import torch.multiprocessing as mp
    world = 2
    with tempfile.TemporaryDirectory() as outdir:
        mp.spawn(_rank, args=(world, _free_port(), outdir), nprocs=world, join=True)
        for c, (scheme, s, q, p) in enumerate(CASES):
            r = [np.load(os.path.join(outdir, f"case{c}_rank{k}.npz")) for k in range(world)]
            nb = r[0]["idx"].size
            assert nb >= 5 and r[1]["idx"].size == nb  # several buckets over three steps
            assert np.array_equal(r[0]["idx"], r[1]["idx"])
            assert np.array_equal(r[0]["seed"], r[1]["seed"])
            assert len(set(r[0]["seed"].tolist())) == nb  # a fresh stream for every reduction
            for k in range(nb):
                x = np.stack([r[0][f"in{k}"], r[1][f"in{k}"]]).astype(np.float32)
                _, _, mean = oracle.compress_mean(x, s, q, p, SCH[scheme], int(r[0]["seed"][k]))
                assert np.array_equal(r[0][f"out{k}"], mean), (c, k)
                assert np.array_equal(r[1][f"out{k}"], mean), (c, k)
            assert np.array_equal(r[0]["grads"], r[1]["grads"])
