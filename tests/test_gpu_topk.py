"""GPU parity: top-k error-feedback encode/decode vs the CPU oracle, bit for bit.

Indices, values, the memory after the step and the decoded vector must match
the oracle exactly (selection order: |acc| descending, index ascending).
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import DEV, TopkRunner, f32_bits, lib, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def one_step(runner, grad_h, mem_h, eta, check_decode=True):
    """Run one encode (+decode) on the GPU and compare with the oracle from the same state."""
    mem_t = to_dev(mem_h.copy())
    runner.encode(to_dev(grad_h), mem_t, eta)
    if check_decode:
        runner.decode()
    ref = oracle.topk_ef_step(mem_h, grad_h, eta, runner.k)
    torch.cuda.synchronize()
    idx = runner.idx.cpu().numpy()
    assert np.array_equal(idx, ref["idx"]), f"indices differ at {np.flatnonzero(idx != ref['idx'])[:10]}"
    assert np.array_equal(f32_bits(runner.val), f32_bits(ref["val"]))
    assert np.array_equal(f32_bits(mem_t), f32_bits(ref["mem"]))
    if check_decode:
        assert np.array_equal(f32_bits(runner.out), f32_bits(oracle.topk_decode(ref["idx"], ref["val"], runner.d)))
    return ref


def test_c1_ten_steps():
    print("case: C1 d=10000 k=100 eta=0.1 x10", flush=True)
    r = TopkRunner(gen.C1_D, gen.C1_K)
    mem_h = np.zeros(gen.C1_D, np.float32)
    mem_t = to_dev(mem_h)
    for t in range(gen.C1_STEPS):
        g = gen.c1_grad(t)
        r.encode(to_dev(g), mem_t, gen.C1_ETA)
        r.decode()
        ref = oracle.topk_ef_step(mem_h, g, gen.C1_ETA, gen.C1_K)
        torch.cuda.synchronize()
        assert np.array_equal(r.idx.cpu().numpy(), ref["idx"])
        assert np.array_equal(f32_bits(r.val), f32_bits(ref["val"]))
        assert np.array_equal(f32_bits(mem_t), f32_bits(ref["mem"]))       # memory carried on the GPU
        assert np.array_equal(f32_bits(r.out), f32_bits(ref["g"]))
        mem_h = ref["mem"]


@pytest.mark.parametrize("d,k", [(1, 1), (3, 2), (4, 4), (4095, 1), (4095, 4095), (4096, 100), (4097, 4097),
                                 (12289, 1000), (12289, 1), (16383, 500), (16384, 16384), (16384, 1), (16385, 163),
                                 (100_003, 777), (300_001, 30_000)])
def test_edge_sizes(d, k):
    print(f"case: edge d={d} k={k}", flush=True)
    g = gen.gaussian_vector(d, d % 1000)
    m = gen.gaussian_vector(d, d % 1000 + 1, 0.5)
    one_step(TopkRunner(d, k), g, m, 0.37)


@pytest.mark.parametrize("d,k", [(16384, 1), (16384, 1234), (16384, 16383), (16385, 1234)])
def test_tie_heavy_single_workgroup_sizes(d, k):
    """Vectors of at most 16384 entries take the single-workgroup encode; the
    first size past it takes the multi-kernel path.  Both on a coarse grid
    (many ties at the threshold), with and without memory, bf16 too."""
    print(f"case: tie-heavy d={d} k={k}", flush=True)
    one_step(TopkRunner(d, k), gen.tie_heavy(d, k), np.zeros(d, np.float32), 1.0)
    one_step(TopkRunner(d, k), gen.tie_heavy(d, k + 1), gen.tie_heavy(d, k + 2), 1.0)
    g = gen.f32_to_bf16_bits(gen.gaussian_vector(d, 40 + k % 7, 1e-3))
    one_step(TopkRunner(d, k), g, gen.gaussian_vector(d, 41, 1e-3), 0.3)


@pytest.mark.parametrize("k", [1, 1000, 12_345, 49_999, 50_000])
def test_tie_heavy(k):
    print(f"case: tie-heavy d=50000 k={k}", flush=True)
    d = 50_000
    one_step(TopkRunner(d, k), gen.tie_heavy(d, k), np.zeros(d, np.float32), 1.0)
    # ties across signs with memory: acc in {+-0.25 j}
    one_step(TopkRunner(d, k), gen.tie_heavy(d, k + 1), gen.tie_heavy(d, k + 2), 1.0)


def test_zero_and_extreme_values():
    print("case: zeros / extremes", flush=True)
    d = 9000
    one_step(TopkRunner(d, 10), np.zeros(d, np.float32), np.zeros(d, np.float32), 1.0)
    r = gen.rng(0, gen.KIND_MISC, 300)
    g = (r.standard_normal(d) * np.exp2(r.integers(-120, 120, d))).astype(np.float32)
    g[::7] = -0.0
    g[::11] = 0.0
    one_step(TopkRunner(d, 500), g, np.zeros(d, np.float32), 1.0)
    one_step(TopkRunner(d, 8000), g, np.zeros(d, np.float32), 0.5)


def test_bf16_gradient():
    print("case: bf16 d=100003 k=1000", flush=True)
    d = 100_003
    g = gen.f32_to_bf16_bits(gen.gaussian_vector(d, 5, 1e-3))
    one_step(TopkRunner(d, 1000), g, gen.gaussian_vector(d, 6, 1e-3), 1.0)


def test_decode_accumulate():
    print("case: decode accumulate", flush=True)
    d, k = 20_000, 300
    run = TopkRunner(d, k)
    g = gen.gaussian_vector(d, 7)
    ref = one_step(run, g, np.zeros(d, np.float32), 1.0, check_decode=False)
    base = gen.gaussian_vector(d, 8)
    run.out.copy_(to_dev(base))
    run.decode(accumulate=True)
    want = oracle.topk_decode(ref["idx"], ref["val"], d, out=base, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(run.out), f32_bits(want))
    # k = 0 decode: all zeros
    gc = lib()
    empty_i = torch.empty(0, dtype=torch.int32, device=DEV)
    empty_v = torch.empty(0, dtype=torch.float32, device=DEV)
    gc.gc_topk_decode(empty_i, empty_v, run.out)
    torch.cuda.synchronize()
    assert not run.out.any().item()


def test_determinism_and_workspace_reuse():
    print("case: determinism + workspace reuse", flush=True)
    d, k = 500_000, 5000
    g = to_dev(gen.gaussian_vector(d, 9))
    m0 = gen.gaussian_vector(d, 10, 0.3)
    run = TopkRunner(d, k)
    outs = []
    for _ in range(2):
        mem = to_dev(m0)
        run.encode(g, mem, 0.9)
        torch.cuda.synchronize()
        outs.append((run.idx.cpu().numpy().copy(), f32_bits(run.val).copy(), f32_bits(mem).copy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
    # the same workspace, reused for a smaller problem
    gc = lib()
    d2, k2 = 70_001, 70
    g2, m2 = gen.gaussian_vector(d2, 11), gen.gaussian_vector(d2, 12)
    idx2 = torch.empty(k2, dtype=torch.int32, device=DEV)
    val2 = torch.empty(k2, dtype=torch.float32, device=DEV)
    mem2 = to_dev(m2)
    gc.gc_topk_ef_encode(to_dev(g2), mem2, 0.5, k2, idx2, val2, run.ws)
    ref = oracle.topk_ef_step(m2, g2, 0.5, k2)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), ref["idx"])
    assert np.array_equal(f32_bits(mem2), f32_bits(ref["mem"]))


@pytest.mark.parametrize("k", gen.C3_KS)
def test_c3_full_size(k):
    """ResNet-50-sized flat gradient, heavy-tailed, at the benchmark's launch shape: 2 steps."""
    print(f"case: C3 d={gen.C3_D} k={k}", flush=True)
    d = gen.C3_D
    run = TopkRunner(d, k)
    mem_h = np.zeros(d, np.float32)
    mem_t = to_dev(mem_h)
    for t in range(2):
        g = gen.c3_grad(t)
        run.encode(to_dev(g), mem_t, 1.0)
        run.decode()
        ref = oracle.topk_ef_step(mem_h, g, 1.0, k)
        torch.cuda.synchronize()
        assert np.array_equal(run.idx.cpu().numpy(), ref["idx"])
        assert np.array_equal(f32_bits(run.val), f32_bits(ref["val"]))
        assert np.array_equal(f32_bits(mem_t), f32_bits(ref["mem"]))
        assert np.array_equal(f32_bits(run.out), f32_bits(ref["g"]))
        mem_h = ref["mem"]


def test_c5_embedding_full_size():
    """BERT-large embedding (30522 x 1024) bf16 gradient, fp32 memory, k = 1%: one step."""
    print("case: C5 embedding bf16 k=312545", flush=True)
    d = gen.BERT_EMB[0] * gen.BERT_EMB[1]
    g = gen.c5_embedding_bf16(0)
    m = gen.gaussian_vector(d, 13, 1e-3)
    one_step(TopkRunner(d, gen.C5_EMB_K), g, m, 1.0)


def test_guess_too_high_takes_full_capture():
    """The sampled guess can only make the capture pass cheaper, never change the
    result: 64 large entries inside one sampled run make the guess exceed the true
    threshold (k = 1000), so the re-reading capture path must run -- bit-exact all the same."""
    d, k = 1 << 20, 1000
    print(f"case: top-k guess above threshold d={d} k={k}", flush=True)
    g = gen.gaussian_vector(d, 77, 1e-3)
    run0 = 5 * (d // 256)                    # start of the 6th sampled run of 64 entries
    g[run0:run0 + 64] = 2.0
    r = TopkRunner(d, k)
    ref = one_step(r, g, np.zeros(d, np.float32), 1.0)
    state = r.ws[:64].view(torch.int32).cpu().numpy()
    assert state[8] == 0, "expected the re-reading capture path (guess above the level-1 bin)"
    assert np.count_nonzero(ref["g"]) == k


def _outside_sampled_runs(d, n, rng):
    """n positions none of which lies in the 256 sampled runs of 64 entries
    (run r starts at floor(r d / 256)), so the sample cannot see them."""
    starts = (np.arange(256, dtype=np.int64) * d) // 256
    pos = []
    while len(pos) < n:
        p = int(rng.integers(0, d))
        r = min(255, (p * 256) // d + 1)
        if not any(s <= p < s + 64 for s in starts[max(0, r - 2):r + 1]):
            pos.append(p)
    return np.unique(np.array(pos, np.int64))


def test_guess_far_below_threshold_scans_up():
    """The k largest magnitudes (around 1e20) all lie outside the sampled runs,
    so the guess comes from the N(0, 1e-3^2) bulk and lies ~1500 level-1 bins
    below the threshold's bin: the slots hold every candidate and the level-1
    bin is found by scanning some 24 windows of 64 bins upwards from the
    guess.  Bit-exact with the oracle."""
    d = 1 << 20
    rng = np.random.default_rng(91)
    g = gen.gaussian_vector(d, 91, 1e-3)
    big = _outside_sampled_runs(d, 3000, rng)
    g[big] = (1e20 * (1.0 + rng.random(big.size))).astype(np.float32) * np.where(rng.random(big.size) < 0.5, -1, 1)
    k = 2000
    print(f"case: top-k guess far below threshold d={d} k={k}", flush=True)
    r = TopkRunner(d, k)
    ref = one_step(r, g, np.zeros(d, np.float32), 1.0)
    state = r.ws[:64].view(torch.int32).cpu().numpy()
    assert state[8] == 1, "expected the slot path (every candidate captured)"
    assert (state[0] - (state[7] >> 19)) > 64 * 10, "guess expected many windows below the level-1 bin"
    assert np.count_nonzero(ref["g"]) == k


def test_guess_far_above_threshold_scans_down():
    """64 entries of 1e30 inside one sampled run lift the guess ~1700 level-1
    bins above the threshold's bin (k = 1000 keeps the sampled rank below 64
    and reaches into the N(0, 1e-3^2) bulk): the capture re-reads the
    accumulator, after finding the level-1 bin by scanning some 27 windows
    downwards from the guess.  Bit-exact."""
    d = 1 << 20
    g = gen.gaussian_vector(d, 92, 1e-3)
    run0 = 7 * (d // 256)
    g[run0:run0 + 64] = 1e30
    k = 1000
    print(f"case: top-k guess far above threshold d={d} k={k}", flush=True)
    r = TopkRunner(d, k)
    ref = one_step(r, g, np.zeros(d, np.float32), 1.0)
    state = r.ws[:64].view(torch.int32).cpu().numpy()
    assert state[8] == 0, "expected the re-reading capture path"
    assert ((state[7] >> 19) - state[0]) > 64 * 10, "guess expected many windows above the level-1 bin"
    assert np.count_nonzero(ref["g"]) == k


def test_max_size():
    """d = INT32_MAX, the longest vector the ABI takes, k = 1%.  The oracle cannot
    run at this size, so the checks are ones that fix the answer:
      * the accumulated values, rebuilt as memory + decoded vector (one of the two
        is +0 at every position), equal the oracle's bit for bit at 2^20 seeded
        positions and at both ends of the vector;
      * indices ascend; every key above the smallest selected key is selected, and
        of the keys equal to it the lowest indices are taken (the unique top-k set
        under |value| descending, index ascending);
      * values, decoded vector and memory agree with that set bit for bit."""
    d = 2**31 - 1
    k = d // 100
    eta = 0.75
    print(f"case: top-k max size d={d} k={k} eta={eta}", flush=True)
    # a seeded normal draw made on the device (a host draw of 2^31 values takes
    # half a minute); the oracle gets the sampled positions of this same tensor
    rng_t = torch.Generator(device=DEV)
    rng_t.manual_seed(91)
    g_t = torch.randn(d, generator=rng_t, dtype=torch.float32, device=DEV).mul_(1e-3)
    rs = np.random.default_rng(5)
    pos = np.unique(np.concatenate([rs.integers(0, d, 1 << 20), np.arange(4096), np.arange(d - 4096, d)]))
    pos_t = torch.from_numpy(pos).to(DEV)
    g_samples = g_t[pos_t].cpu().numpy()
    mem_t = torch.zeros(d, dtype=torch.float32, device=DEV)
    r = TopkRunner(d, k)
    r.encode(g_t, mem_t, eta)
    r.decode()
    torch.cuda.synchronize()
    del g_t
    acc = mem_t + r.out
    want = oracle.ef_accumulate(np.zeros(pos.size, np.float32), g_samples, eta)
    assert np.array_equal(f32_bits(acc[pos_t]), f32_bits(want))

    idx = r.idx.long()
    assert int(idx[0]) >= 0 and int(idx[-1]) < d and bool((idx[1:] > idx[:-1]).all())
    key = acc.view(torch.int32) & 0x7FFFFFFF
    ksel = key[idx]
    thr = int(ksel.min())
    n_gt = int((key > thr).sum())
    assert int((ksel > thr).sum()) == n_gt
    ties = torch.nonzero(key == thr).flatten()
    n_take = k - n_gt
    assert 1 <= n_take <= ties.numel()
    assert torch.equal(idx[ksel == thr], ties[:n_take])
    del key, ksel, ties

    assert torch.equal(r.val.view(torch.int32), acc[idx].view(torch.int32))
    assert bool((mem_t[idx].view(torch.int32) == 0).all())
    assert int((r.out != 0).sum()) == k
    del acc, idx, mem_t, r
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_random_sizes(seed):
    """Seeded random (d, k) from 1 to 3M, bit-exact: tile tails, tiny and huge k."""
    rs = np.random.default_rng(200 + seed)
    d = int(rs.choice([rs.integers(1, 5000), rs.integers(5000, 200_000), rs.integers(200_000, 3_000_000)]))
    k = int(rs.choice([1, rs.integers(1, d + 1), max(1, d // 100), d]))
    print(f"case: random top-k seed={seed} d={d} k={k}", flush=True)
    g = gen.gaussian_vector(d, 400 + seed, 1e-3)
    m = gen.gaussian_vector(d, 500 + seed, 1e-3)
    one_step(TopkRunner(d, k), g, m, 0.5)
