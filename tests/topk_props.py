"""Properties that fix one exact top-k error-feedback step ("Sparsified SGD
with Memory", method section), checked with torch ops on whatever device the
tensors live on, so they apply at sizes the oracle cannot reach."""
import torch


def check_topk_step_properties(acc, idx, val, out, mem_after, k, label):
    """What fixes one exact top-k EF step at any size, checked on the device:
    the k indices ascend; every selected key (|acc| bits) is >= every other
    key, and among keys equal to the smallest selected one the lowest indices
    are taken; the values are acc's entries bit for bit; the decode is zero
    except at the pairs; the memory is acc with the selected entries +0.0."""
    assert idx.numel() == k
    idx64 = idx.long()
    assert bool((idx64[1:] > idx64[:-1]).all()), f"{label}: indices not strictly ascending"
    key = acc.view(torch.int32) & 0x7FFFFFFF
    sel = torch.zeros(acc.numel(), dtype=torch.bool, device=acc.device)
    sel[idx64] = True
    thr = key[idx64].min()
    if k < acc.numel():
        assert int(key[~sel].max()) <= int(thr), f"{label}: an unselected key exceeds a selected one"
    ties = torch.nonzero(key == thr).flatten()
    taken = int(sel[ties].sum())
    assert bool(sel[ties[:taken]].all()), f"{label}: ties not taken lowest index first"
    assert torch.equal(val.view(torch.int32), acc[idx64].view(torch.int32)), f"{label}: values differ from acc"
    want_out = torch.zeros_like(acc)
    want_out[idx64] = val
    assert torch.equal(out.view(torch.int32), want_out.view(torch.int32)), f"{label}: decode"
    want_mem = acc.clone()
    want_mem[idx64] = 0.0
    assert torch.equal(mem_after.view(torch.int32), want_mem.view(torch.int32)), f"{label}: memory"
