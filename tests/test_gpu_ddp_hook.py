"""The DDP communication hook on one MI355X, with one rank over RCCL.

A model's gradient buckets (25 MB by default) go through
`global_qsgd_hook` and the HIP library during backward. The hook runs the
norm term, an all-reduce of it, N, the codes in the word layout, an integer
all-reduce and dequantization. With one rank each bucket is one worker, so
every bucket's mean must equal the oracle's `compress_mean` of that bucket
as a [1, d] input with the seed the hook used, bit for bit. The test covers
two schemes, two steps, and the gradients DDP writes back.
"""
import math
import os
import socket
import sys
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")
import torch.distributed as dist  # noqa: E402

import allreduce_compatible_gradient_amd as gq  # noqa: E402
import oracle  # noqa: E402

pytestmark = pytest.mark.gpu
SCH = {"L": oracle.SCHEME_L, "E": oracle.SCHEME_E}


def log(msg):
    print(f"[gpu-ddp {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def one_rank_group():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.lib()
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        port = s.getsockname()[1]
    torch.cuda.set_device(0)
    dist.init_process_group("nccl", init_method=f"tcp://127.0.0.1:{port}", rank=0, world_size=1)
    yield
    dist.destroy_process_group()


@pytest.mark.parametrize("scheme,s,q,p", [("L", 127, 2.0, math.inf), ("E", 8, 2.0, 2.0)])
def test_hook_buckets_match_the_oracle(one_rank_group, scheme, s, q, p):
    from torch.nn.parallel import DistributedDataParallel as DDP

    from allreduce_compatible_gradient_amd.ddp import GlobalQSGDState, global_qsgd_hook
    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(2048, 2048), torch.nn.Tanh(),
                                torch.nn.Linear(2048, 2048), torch.nn.Tanh(),
                                torch.nn.Linear(2048, 1536)).cuda()
    ddp = DDP(model, device_ids=[0])  # default 25 MB buckets
    state = GlobalQSGDState(scheme=scheme, s=s, q=q, p=p, seed=11)
    seeds, recs = [], []
    plain_next = state.next_seed

    def next_seed(i):
        sd = plain_next(i)
        seeds.append(sd)
        return sd
    state.next_seed = next_seed

    def hook(st, bucket):
        inp = bucket.buffer().detach().clone()
        fut = global_qsgd_hook(st, bucket)
        sd = seeds[-1]

        def keep(f):
            recs.append((bucket.index(), inp, f.value().detach().clone(), sd))
            return f.value()
        return fut.then(keep)
    ddp.register_comm_hook(state, hook)
    g = torch.Generator(device="cuda").manual_seed(5)
    for _ in range(2):
        ddp.zero_grad()
        x = torch.randn(64, 2048, device="cuda", generator=g)
        ddp(x).pow(2).mean().backward()
    torch.cuda.synchronize()
    assert len(recs) >= 3 and len(set(r[3] for r in recs)) == len(recs)
    for idx, inp, out, sd in recs:
        xin = inp.cpu().numpy().reshape(1, -1)
        N, _, mean = oracle.compress_mean(xin, s, q, p, SCH[scheme], sd)
        assert np.array_equal(out.cpu().numpy(), mean), (idx, xin.size)
        log(f"{scheme} s={s}: bucket {idx}, {xin.size} gradients ({4 * xin.size / 2**20:.1f} MB), "
            f"N = {float(N):.6g}: mean bit-exact")
    # the gradients DDP wrote back are the last step's bucket means
    last = {}
    for idx, _, out, _ in recs:
        last[idx] = out
    total = sum(prm.numel() for prm in model.parameters())
    assert sum(o.numel() for o in last.values()) == total
    got = np.sort(np.concatenate([prm.grad.detach().cpu().numpy().ravel()
                                  for prm in model.parameters()]))
    want = np.sort(np.concatenate([o.cpu().numpy() for o in last.values()]))
    assert np.array_equal(got, want)


class _Bucket:
    """The part of DDP's GradBucket the hook reads."""

    def __init__(self, buf, index):
        self._buf, self._index = buf, index

    def buffer(self):
        return self._buf

    def index(self):
        return self._index


@pytest.mark.parametrize("scheme,s,q,p", [("L", 15, 2.0, 2.0), ("E", 8, math.inf, 2.0)])
def test_hook_on_a_bf16_bucket(one_rank_group, scheme, s, q, p):
    """A bf16 gradient bucket (a bf16 model's): the codes come from the
    bf16 values widened exactly, the mean is formed in fp32 and written back
    rounded to bf16 (to nearest, ties to even) -- the oracle's mean rounded
    the same way, bit for bit.  Two calls on one bucket use two seeds."""
    import workloads as wl

    from allreduce_compatible_gradient_amd.ddp import GlobalQSGDState, global_qsgd_hook
    d = 3_000_017
    x = wl.random_rows(1, d, seed=21, dtype="bf16", scale=0.02)
    state = GlobalQSGDState(scheme=scheme, s=s, q=q, p=p, seed=3)
    seeds = []
    plain_next = state.next_seed

    def next_seed(i):
        seeds.append(plain_next(i))
        return seeds[-1]
    state.next_seed = next_seed
    for call in range(2):
        buf = torch.from_numpy(x.view(np.int16).copy()).to("cuda").view(torch.bfloat16)[0]
        out = global_qsgd_hook(state, _Bucket(buf, 4)).wait()
        torch.cuda.synchronize()
        _, _, mean = oracle.compress_mean(x, s, q, p, SCH[scheme], seeds[-1])
        want = wl.f32_to_bf16_bits(mean)
        assert out.dtype == torch.bfloat16
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), want), call
    assert seeds[0] != seeds[1]
