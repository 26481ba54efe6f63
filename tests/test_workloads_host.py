"""The seeded generators do their per-row work on the host: a block table or index list reaches
its device with one copy, never through per-row device writes. Checked on the "meta" device,
where every operation that touches a device tensor is visible to a dispatch mode; the generators
hold no method arithmetic, so only their data movement is checked here (plus their contracts)."""

import torch
from torch.utils._python_dispatch import TorchDispatchMode

from nvfp4_compressed_mla_amd import workloads as wl


class _DeviceOps(TorchDispatchMode):
    def __init__(self):
        super().__init__()
        self.ops = []

    def __torch_dispatch__(self, func, types, args=(), kwargs=None):
        kwargs = kwargs or {}
        flat = [a for a in list(args) + list(kwargs.values())]
        out = func(*args, **kwargs)
        outs = out if isinstance(out, (tuple, list)) else [out]
        touched = [t for t in flat + list(outs) if isinstance(t, torch.Tensor) and t.device.type == "meta"]
        if touched or kwargs.get("device") == torch.device("meta"):
            self.ops.append(str(func))
        return out


def _count(fn):
    mode = _DeviceOps()
    with mode:
        res = fn()
    return res, mode.ops


def test_block_table_one_copy():
    (bt, total), ops = _count(lambda: wl.gen_block_table([300, 64, 1000, 5], 3, "meta", spare_pages=2))
    assert bt.device.type == "meta" and tuple(bt.shape) == (4, 16) and total == 5 + 1 + 16 + 1 + 2
    assert len(ops) == 1, ops


def test_topk_lists_one_copy():
    idx, ops = _count(lambda: wl.gen_topk(3, 4, 64, [1000, 30, 64], 5, "meta", q_lens=[4, 2, 1]))
    assert idx.device.type == "meta" and tuple(idx.shape) == (3, 4, 64)
    assert len(ops) == 1, ops
    idx, ops = _count(lambda: wl.gen_topk_overlap(2, 5, 32, [500, 400], 0.5, 6, "meta"))
    assert idx.device.type == "meta" and len(ops) == 1, ops


def test_topk_list_contracts_on_host():
    idx = wl.gen_topk(3, 4, 64, [1000, 30, 64], 5, "cpu", q_lens=[4, 2, 1])
    for b, (c, nq) in enumerate(zip([1000, 30, 64], [4, 2, 1])):
        for t in range(4):
            row = idx[b, t]
            if t >= nq:
                assert torch.all(row == -1)
                continue
            v = row[row >= 0]
            assert v.numel() == min(c, 64) and torch.unique(v).numel() == v.numel()
            assert int(v.max()) < c
    ov = wl.gen_topk_overlap(2, 5, 32, [500, 400], 0.5, 6, "cpu")
    for b in range(2):
        base = set(ov[b, 0].tolist())
        for t in range(5):
            row = ov[b, t].tolist()
            assert row == sorted(row) and len(set(row)) == 32
    assert torch.equal(wl.gen_topk(2, 2, 16, [100, 50], 9), wl.gen_topk(2, 2, 16, [100, 50], 9))
