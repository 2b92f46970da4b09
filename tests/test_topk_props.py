"""CPU: the top-k step property check has teeth.  A correct step (the
oracle's) passes; each planted mistake in it fails: a swapped selected and
unselected entry, ties taken from the top, a value off by one ulp, a decode
entry missing, a selected memory entry not zeroed, indices out of order."""
import numpy as np
import pytest
import torch

import gen
import oracle
from topk_props import check_topk_step_properties


def case(d=5000, k=60, ties=True):
    acc = gen.gaussian_vector(d, 11, 1.0)
    if ties:
        acc[100:140] = 2.5        # 40 equal keys that straddle the threshold
        acc[200:210] = -2.5
    ref = oracle.topk_ef_step(np.zeros(d, np.float32), acc, 1.0, k)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    out = oracle.topk_decode(ref["idx"], ref["val"], d)
    return t(acc), t(ref["idx"].astype(np.int32)), t(ref["val"]), t(out), t(ref["mem"]), k


def test_correct_step_passes():
    acc, idx, val, out, mem, k = case()
    check_topk_step_properties(acc, idx, val, out, mem, k, "oracle step")


def planted(kind):
    acc, idx, val, out, mem, k = case()
    idx, val, out, mem = idx.clone(), val.clone(), out.clone(), mem.clone()
    if kind == "swap":
        # replace the smallest selected entry by the largest unselected one
        sel = torch.zeros(acc.numel(), dtype=torch.bool)
        sel[idx.long()] = True
        key = acc.view(torch.int32) & 0x7FFFFFFF
        lo = idx[torch.argmin(key[idx.long()])].item()
        cand = torch.nonzero(~sel).flatten()
        hi = cand[torch.argmax(key[cand])].item()
        if key[hi] == key[lo]:
            cand = cand[key[cand] < key[lo]]
            hi = cand[torch.argmax(key[cand])].item()
        new = sorted(set(idx.tolist()) - {lo} | {hi})
        idx = torch.tensor(new, dtype=torch.int32)
        val = acc[idx.long()].clone()
        out = torch.zeros_like(acc)
        out[idx.long()] = val
        mem = acc.clone()
        mem[idx.long()] = 0.0
    elif kind == "tie_order":
        key = acc.view(torch.int32) & 0x7FFFFFFF
        thr = key[idx.long()].min()
        ties = torch.nonzero(key == thr).flatten().tolist()
        taken = [i for i in ties if i in set(idx.tolist())]
        assert 0 < len(taken) < len(ties)
        swap_out, swap_in = taken[0], ties[-1]
        new = sorted(set(idx.tolist()) - {swap_out} | {swap_in})
        idx = torch.tensor(new, dtype=torch.int32)
        val = acc[idx.long()].clone()
        out = torch.zeros_like(acc)
        out[idx.long()] = val
        mem = acc.clone()
        mem[idx.long()] = 0.0
    elif kind == "value_ulp":
        val[3] = torch.from_numpy(np.nextafter(val[3:4].numpy(), np.float32(np.inf)))[0]
    elif kind == "decode_missing":
        out[idx[5].long()] = 0.0
    elif kind == "memory_not_zeroed":
        mem[idx[7].long()] = acc[idx[7].long()]
    elif kind == "order":
        idx = idx.flip(0)
        val = val.flip(0)
    return acc, idx, val, out, mem, k


@pytest.mark.parametrize("kind", ["swap", "tie_order", "value_ulp", "decode_missing", "memory_not_zeroed", "order"])
def test_planted_mistake_fails(kind):
    with pytest.raises(AssertionError):
        check_topk_step_properties(*planted(kind), kind)
