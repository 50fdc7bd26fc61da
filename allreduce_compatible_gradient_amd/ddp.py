"""Global-QSGD as a DistributedDataParallel communication hook.

"Global-QSGD: Practical Floatless Quantization for Distributed Learning with
Theoretical Guarantees", Sec. 6 (implementation): the operator runs inside
a DDP communication hook. DDP calls it once per gradient bucket (25 MB by
default), and it quantizes, all-reduces and dequantizes. Here each rank is
one worker, its bucket one row of the operator's input. Per bucket:

1. The norm. `gq_norm_term` gives the rank's fp64 term (sum of squares for
   q = 2, max |x| for q = inf, combined over its row as the norm takes it
   before its root). One `all_reduce` of that double combines the terms:
   SUM for finite p, MAX for p = inf. `gq_norm_from_term` then gives the
   global N, the same bits on every rank.
2. The codes. `gq_quantize_words` writes the rank's codes at worker index
   `rank` (the Philox counter carries it), in the word layout. That layout
   puts floor(32 / W) fields of code + M in each 32-bit word. W is the
   minimal width for `world` workers, so a native integer SUM of the words
   adds the codes exactly and never carries between fields.
3. The integer all-reduce. One `all_reduce` (SUM) of the int32 words. It is
   exact and independent of the collective's algorithm or order, since
   two's-complement int32 addition is the uint32 sum modulo 2^32.
4. Dequantization. `gq_dequantize_words` with n = world gives the mean
   gradient, which DDP writes into the parameters' gradients.

Every step is enqueued in stream order: each collective makes the current
stream wait for it, and the host never blocks. The returned future is
already complete, and on a GPU it carries the current stream's events.

The arithmetic of every step runs in libgq.so's kernels. This module only
orders the calls and the two collectives, and derives each call's Philox
seed. The seed comes from (base seed, bucket index, how many times that
bucket has been reduced), the same on every rank, so no two reductions
reuse a random stream.

`ops` exists so that the multi-rank orchestration can be tested on CPUs
(gloo) with stand-ins for the four library calls. The default is the HIP
library, and nothing else runs on a GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from types import SimpleNamespace

import torch
import torch.distributed as dist

from . import (gq_dequantize_words, gq_min_code_bits, gq_norm_from_term, gq_norm_term,
               gq_quantize_words, gq_word_row_bytes, gq_workspace_bytes)

_MASK64 = (1 << 64) - 1


def _mix64(v: int) -> int:
    """splitmix64 finalizer (Steele, Lea, Flood, "Fast splittable pseudorandom
    number generators", OOPSLA 2014): spreads a 64-bit counter over the key."""
    v = (v + 0x9E3779B97F4A7C15) & _MASK64
    v = ((v ^ (v >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    v = ((v ^ (v >> 27)) * 0x94D049BB133111EB) & _MASK64
    return v ^ (v >> 31)


def library_ops():
    """The four device calls of the hook: libgq.so through the binding."""
    return SimpleNamespace(norm_term=gq_norm_term, norm_from_term=gq_norm_from_term,
                           quantize_words=gq_quantize_words,
                           dequantize_words=gq_dequantize_words)


@dataclass
class GlobalQSGDState:
    """Settings of the hook and its per-bucket call counters.

    scheme, s: Global-L_s ("L", levels (s-i)/s) or Global-E_s ("E", levels
    2^-k); q, p: the (q,p)-norm (q within a rank's bucket, p over the
    ranks); seed: base key of the Philox streams."""
    scheme: str = "L"
    s: int = 127
    q: float = 2.0
    p: float = math.inf
    seed: int = 0
    process_group: object = None
    ops: object = None
    calls: dict = field(default_factory=dict)
    buffers: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.ops is None:
            self.ops = library_ops()

    def bucket_buffers(self, bucket_index: int, buf: torch.Tensor, W: int):
        """Device buffers of one bucket's reduction, kept between calls: the
        norm term, N, the norm pass's workspace and the word row.  Reuse is
        ordered by the stream: a bucket's next codes are written after its
        previous dequantization, which waits for the all-reduce that read
        the words."""
        d = buf.numel()
        key = (bucket_index, d, buf.dtype, buf.device, W)
        b = self.buffers.get(key)
        if b is None:
            dev = buf.device
            b = SimpleNamespace(
                term=torch.empty(1, dtype=torch.float64, device=dev),
                norm=torch.empty(1, dtype=torch.float32, device=dev),
                ws=torch.empty(max(gq_workspace_bytes(1, d), 16), dtype=torch.uint8, device=dev)
                if dev.type == "cuda" else None,
                words=torch.empty((1, max(gq_word_row_bytes(d, W), 16) // 4), dtype=torch.int32,
                                  device=dev) if dev.type == "cuda" else None)
            self.buffers = {k: v for k, v in self.buffers.items() if k[0] != bucket_index}
            self.buffers[key] = b
        return b

    def next_seed(self, bucket_index: int) -> int:
        """Philox key of this reduction of the bucket: distinct for every
        (bucket, call), identical on every rank."""
        k = self.calls.get(bucket_index, 0)
        self.calls[bucket_index] = k + 1
        return _mix64(_mix64(self.seed ^ (bucket_index << 40)) ^ k)


def global_qsgd_hook(state: GlobalQSGDState, bucket) -> torch.futures.Future:
    """DDP communication hook (register with `ddp.register_comm_hook(state,
    global_qsgd_hook)`): the bucket's mean gradient over the ranks, through
    Global-Q codes and an integer all-reduce."""
    group = state.process_group if state.process_group is not None else dist.group.WORLD
    world = dist.get_world_size(group)
    rank = dist.get_rank(group)
    ops = state.ops
    buf = bucket.buffer()
    x = buf.view(1, -1)
    d = x.shape[1]
    W = gq_min_code_bits(world, state.s, state.scheme)
    if W < 0 or W > 32:
        raise ValueError(f"sums of {world} codes with s = {state.s} do not fit 32 bits")
    bb = state.bucket_buffers(bucket.index(), buf, W)
    # 1. global norm: each rank's term, one all-reduce of a double
    term = ops.norm_term(x, state.q, state.p, term=bb.term, workspace=bb.ws)
    dist.all_reduce(term, op=dist.ReduceOp.MAX if math.isinf(state.p) else dist.ReduceOp.SUM,
                    group=group)
    norm = ops.norm_from_term(term, state.q, state.p, norm=bb.norm)
    # 2. this rank's codes in the word layout, at its worker index
    words = ops.quantize_words(x, state.s, state.scheme, norm, state.next_seed(bucket.index()),
                               W, worker_base=rank, words=bb.words)[0]
    # 3. the integer all-reduce of the codes, ordered on the current stream
    #    like the norm term's (the host does not wait for it)
    dist.all_reduce(words, op=dist.ReduceOp.SUM, group=group)
    # 4. one dequantization to the mean, written into the bucket after it
    if buf.dtype == torch.float32:
        ops.dequantize_words(words, world, d, state.s, state.scheme, W, norm, mean=buf)
    else:
        buf.copy_(ops.dequantize_words(words, world, d, state.s, state.scheme, W, norm))
    # a future already holding the bucket; on a GPU it records the current
    # stream, so whoever waits on it waits for the work above (a continuation
    # on the all-reduce's own future measured 57 against 9 us of host time)
    fut = torch.futures.Future(devices=[buf.device]) if buf.is_cuda else torch.futures.Future()
    fut.set_result(buf)
    return fut
