"""GPU parity of the cross-entropy path against the CPU oracle (bit-exact) and
the properties of the det-cross-entropy page ("Correctness": vocabulary splits
2/4/8 give loss, denominator and gradient torch.equal to the single call;
repeated forward and backward passes are bitwise identical)."""
import sys

import numpy as np
import pytest
import torch

from bitwise_deterministic_exact_pass1_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def CE():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from bitwise_deterministic_exact_pass1_amd import cross_entropy
    return cross_entropy


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def u32(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


@pytest.fixture(scope="module")
def vocab(CE):
    say("ce: inputs N=4096 V=128256 bf16")
    x, t = W.ce_inputs()
    X, T = x.cuda(), t.cuda()
    loss, m, denom = CE.forward(X, T)
    torch.cuda.synchronize()
    return x, t, X, T, loss, m, denom


def test_forward_bit_exact_full_vocab(vocab, oracle):
    x, t, X, T, loss, m, denom = vocab
    say("ce: oracle forward (full)")
    rl, rm, rd = oracle.ce_forward(x, t)
    assert np.array_equal(u32(m), u32(rm))
    assert np.array_equal(denom.cpu().numpy(), rd)
    assert np.array_equal(u32(loss), u32(rl))


def test_reductions_bit_exact(CE, vocab, oracle):
    x, t, X, T, loss, m, denom = vocab
    l = loss.cpu().numpy()
    for red in ("mean", "sum"):
        assert u32(CE.reduce(loss, red).reshape(1)) == u32(np.float32(oracle.ce_reduce(l, red)))
    assert torch.equal(CE.reduce(loss, "none"), loss)


@pytest.mark.parametrize("reduction", ["none", "mean", "sum"])
def test_gradient_bit_exact_sampled_rows(CE, vocab, oracle, reduction):
    x, t, X, T, loss, m, denom = vocab
    g = torch.full((4096,), 0.75) if reduction == "none" else torch.tensor([1.25])
    grad = CE.backward(X, T, m, denom, g.cuda(), reduction)
    rows = np.array([0, 1, 777, 2048, 4095])
    xs = x[rows].contiguous()
    gs = g[rows] if reduction == "none" else g
    mr, dr = m.cpu().numpy()[rows], denom.cpu().numpy()[rows]
    if reduction == "mean":  # c = RN64(g / N) uses the full batch N = 4096
        ref = oracle_mean_rows(oracle, xs, t[rows], mr, dr, 1.25, 4096)
    else:
        ref = oracle.ce_backward(xs, t[rows], mr, dr, gs.numpy(), reduction)
    assert np.array_equal(u32(grad.cpu().numpy()[rows]), u32(ref))


def oracle_mean_rows(oracle, xs, ts, m, d, g, N):
    """Mean-reduction gradient rows of an N-row batch, from the oracle's
    'none' path with every row's upstream set to c = RN64(g/N); N is a power of
    two here, so c is exact and an f32 carries it unchanged."""
    c = np.float32(g / N)
    assert float(c) == g / N
    return oracle.ce_backward(xs, ts, m, d, np.full(len(xs), c, np.float32), "none")


def test_gradient_bit_exact_all_rows_mean(CE, vocab, oracle):
    """The whole [4096, 128256] gradient of the mean loss (upstream 1) against
    the oracle, every element."""
    x, t, X, T, loss, m, denom = vocab
    say("ce: full gradient (mean) on the GPU")
    grad = CE.backward(X, T, m, denom, torch.ones(1).cuda(), "mean").cpu().numpy()
    say("ce: full gradient (mean) in the oracle")
    ref = oracle.ce_backward(x, t, m.cpu().numpy(), denom.cpu().numpy(), np.ones(1, np.float32), "mean")
    assert np.array_equal(u32(grad), u32(ref))


@pytest.mark.parametrize("nsplit", [2, 4, 8])
def test_vocab_shard_gradients_compose_bit_exact(CE, vocab, nsplit):
    """Each vocabulary shard's gradient (its columns as a view, targets as
    whole-vocabulary indices, the composed rowmax and denominator) is that
    shard's columns of the whole gradient, torch.equal, for every reduction."""
    x, t, X, T, loss, m, denom = vocab
    V = X.shape[1]
    bounds = np.linspace(0, V, nsplit + 1).astype(int).tolist()
    for reduction, g in (("mean", torch.ones(1)), ("sum", torch.tensor([0.5])), ("none", torch.full((4096,), 0.75))):
        whole = CE.backward(X, T, m, denom, g.cuda(), reduction)
        parts = [CE.backward(X[:, lo:hi], T, m, denom, g.cuda(), reduction, v0=lo)
                 for lo, hi in zip(bounds[:-1], bounds[1:])]
        assert torch.equal(torch.cat(parts, 1), whole), (nsplit, reduction)
        del whole, parts


@pytest.mark.parametrize("nsplit", [1, 2, 4, 8])
def test_vocab_split_invariance(CE, vocab, nsplit):
    x, t, X, T, loss, m, denom = vocab
    V = X.shape[1]
    bounds = np.linspace(0, V, nsplit + 1).astype(int)
    shards = list(zip(bounds[:-1].tolist(), bounds[1:].tolist()))
    order = W.shard_order(4000 + nsplit, nsplit)
    gm = torch.stack([CE.rowmax(X, lo, hi) for lo, hi in shards]).amax(0)
    assert torch.equal(gm, m)
    den = None
    for s in order:
        lo, hi = shards[s]
        den = CE.denom_digits(X, gm, lo, hi) if den is None else CE.denom_digits(X, gm, lo, hi, out=den)
    l2, d2 = CE.finalize(den, X, T, gm)
    assert torch.equal(l2, loss) and torch.equal(d2, denom)
    # the page's caller-side composition: a plain int64 sum of per-shard digits
    den_sum = sum(CE.denom_digits(X, gm, lo, hi) for lo, hi in shards)
    l3, d3 = CE.finalize(den_sum, X, T, gm)
    assert torch.equal(l3, loss) and torch.equal(d3, denom)


def test_autograd_deterministic(CE, vocab):
    x, t, X, T, loss, m, denom = vocab
    Xs = X[:512].clone().requires_grad_(True)
    Ts = T[:512]
    outs = []
    for _ in range(2):
        Xs.grad = None
        l = CE.cross_entropy(Xs, Ts, reduction="mean")
        l.backward()
        outs.append((l.detach().clone(), Xs.grad.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert outs[0][1].dtype == torch.bfloat16
    ref = torch.nn.functional.cross_entropy(Xs.detach().double().cpu(), Ts.cpu())
    assert abs(float(outs[0][0]) - float(ref)) <= 2e-6


def test_f32_logits_small(CE, oracle):
    x, t = W.ce_inputs(seed=44, N=33, V=1000, dtype=torch.float32)
    loss, m, denom = CE.forward(x.cuda(), t.cuda())
    rl, rm, rd = oracle.ce_forward(x, t)
    assert np.array_equal(u32(loss), u32(rl)) and np.array_equal(denom.cpu().numpy(), rd)
    g = CE.backward(x.cuda(), t.cuda(), m, denom, torch.ones(1).cuda(), "sum")
    ref = oracle.ce_backward(x, t, rm, rd, np.ones(1, np.float32), "sum")
    assert np.array_equal(u32(g), u32(ref))


def edge_logits():
    """bf16 rows that reach every branch of the pattern-table kernels: a row view
    with an odd row stride and a start offset of 3 (scalar heads and tails), rows
    whose maximum is negative, +0 or -0, rows with most patterns outside the
    32-binade window (the out-of-window queue overflows and the row is scanned
    again), a few outliers (queue without overflow), tiny magnitudes, weights
    that underflow to zero, constant rows, and targets in the head and tail."""
    g = torch.Generator().manual_seed(46)
    N, V = 16, 20011
    big = torch.randn(N, V + 8, generator=g) * 2.0
    x = big[:, 3:3 + V]
    x[1] = -x[1].abs() - 1.0
    x[2] = -x[2].abs()
    x[2, 100:140] = -0.0
    x[2, 7777] = 0.0
    x[3] = -x[3].abs()
    x[3, 5000:5010] = -0.0
    e = torch.randint(-60, 12, (V,), generator=g).float()
    s = torch.where(torch.rand(V, generator=g) < 0.5, -1.0, 1.0)
    x[4] = s * torch.exp2(e) * (1 + torch.rand(V, generator=g))
    x[5] = torch.randn(V, generator=g)
    idx = 3000 + torch.randperm(V - 3000, generator=g)[:100]   # beyond the sampled first vectors
    x[5, idx] = torch.where(torch.rand(100, generator=g) < 0.5, -1.0, 1.0) * torch.exp2(
        torch.randint(8, 14, (100,), generator=g).float())
    x[6] = torch.randn(V, generator=g) * 2.0 ** -40
    x[6, :7] = torch.randn(7, generator=g)
    x[7] = torch.randn(V, generator=g) * 200.0
    x[8] = 1.5
    x[9, 0] = 40.0
    x[10, V - 1] = 40.0
    xb = big.to(torch.bfloat16)[:, 3:3 + V]
    t = torch.randint(0, V, (N,), generator=g)
    t[9], t[10], t[11] = 0, V - 1, 2
    return xb, t


@pytest.fixture(scope="module")
def edge(CE):
    say("ce: edge rows N=16 V=20011 bf16, row stride 20019, offset 3")
    x, t = edge_logits()
    assert x.stride(0) == 20019 and x.storage_offset() == 3
    return x, t, x.cuda(), t.cuda()


def test_pattern_tables_forward_edge_rows(CE, edge, oracle):
    x, t, X, T = edge
    loss, m, denom = CE.forward(X, T)
    rl, rm, rd = oracle.ce_forward(x, t)
    assert np.array_equal(u32(m), u32(rm))
    assert np.array_equal(denom.cpu().numpy(), rd)
    assert np.array_equal(u32(loss), u32(rl))
    assert u32(m)[2] == 0 and u32(m)[3] == 0x80000000  # +0 and -0 maxima


def test_pattern_tables_split_digits_edge_rows(CE, edge, oracle):
    x, t, X, T = edge
    V = X.shape[1]
    shards = [(0, 8203), (8203, 16411), (16411, V)]   # 8203 and 8208 long: both use the tables
    ms = [CE.rowmax(X, lo, hi) for lo, hi in shards]
    for (lo, hi), mm in zip(shards, ms):
        assert np.array_equal(u32(mm), u32(oracle.ce_rowmax(x, lo, hi)))
    gm = torch.stack(ms).amax(0)
    loss, m, denom = CE.forward(X, T)
    assert torch.equal(gm, m)
    den = None
    for lo, hi in shards:
        part = CE.denom_digits(X, gm, lo, hi)
        assert np.array_equal(part.cpu().numpy(), oracle.ce_denom_digits(x, gm.cpu().numpy(), lo, hi))
        den = CE.denom_digits(X, gm, lo, hi) if den is None else CE.denom_digits(X, gm, lo, hi, out=den)
    l2, d2 = CE.finalize(den, X, T, gm)
    assert torch.equal(l2, loss) and torch.equal(d2, denom)


def test_pattern_tables_gradient_edge_rows(CE, edge, oracle):
    x, t, X, T = edge
    loss, m, denom = CE.forward(X, T)
    g = torch.linspace(-1.5, 1.5, X.shape[0])  # negative upstream values give -0 gradients
    grad = CE.backward(X, T, m, denom, g.cuda(), "none")
    ref = oracle.ce_backward(x, t, m.cpu().numpy(), denom.cpu().numpy(), g.numpy(), "none")
    assert np.array_equal(u32(grad.cpu().numpy()), u32(ref))


@pytest.mark.parametrize("nvec", [1900, 2004, 2047, 2048, 2100, 3584, 3585, 3700, 4000, 4095, 4096, 5000])
def test_range_lengths_around_the_first_load_batch(CE, oracle, nvec):
    """Ranges of 8 * nvec bf16 columns, around eight 16-byte vectors per thread
    of a 512-thread row workgroup (where the row kernels switch between placing
    the window from a first load batch and from a separate sample), and
    shorter ones: forward and denominator digits equal the oracle bit for bit."""
    x, t = W.ce_inputs(seed=47, N=24, V=8 * nvec)
    X, T = x.cuda(), t.cuda()
    loss, m, denom = CE.forward(X, T)
    rl, rm, rd = oracle.ce_forward(x, t)
    assert np.array_equal(u32(loss), u32(rl)) and np.array_equal(denom.cpu().numpy(), rd)
    lo = 8 * (nvec // 3)
    d = CE.denom_digits(X, m, lo, 8 * nvec).cpu().numpy()
    ref = oracle.ce_denom_digits(x, m.cpu().numpy(), lo, 8 * nvec)
    val = lambda a: [sum(int(a[k, i]) << (32 * k) for k in range(a.shape[0])) for i in range(a.shape[1])]
    assert val(d) == val(ref)


def test_pattern_counts_past_16_bits(CE, oracle):
    """Rows where one bf16 pattern occurs more than 65535 times, beside rows of
    two patterns of 35000 each: forward, split denominator digits and
    gradient equal the oracle bit for bit (the pattern counts times the
    pattern weights stay exact at any count the tables admit)."""
    g = torch.Generator().manual_seed(48)
    N, V = 4, 70001
    x = (torch.randn(N, V, generator=g) * 2.0)
    x[0] = 0.5                        # one pattern everywhere
    x[1, :66000] = -1.25              # 66000 copies beside random values
    x[2, :35000] = 1.0                # two patterns of 35000, no overflow
    x[2, 35000:70000] = -1.0
    x[3, 100:65737] = 3.0             # exactly 65637 copies, beside the row max
    x = x.to(torch.bfloat16)
    t = torch.tensor([5, 66001, 12, 70000], dtype=torch.int64)
    X, T = x.cuda(), t.cuda()
    loss, m, denom = CE.forward(X, T)
    rl, rm, rd = oracle.ce_forward(x, t)
    assert np.array_equal(u32(loss), u32(rl)) and np.array_equal(denom.cpu().numpy(), rd)
    assert np.array_equal(u32(m), u32(rm))
    for lo, hi in [(0, V), (1000, V)]:
        d = CE.denom_digits(X, m, lo, hi).cpu().numpy()
        ref = oracle.ce_denom_digits(x, m.cpu().numpy(), lo, hi)
        val = lambda a: [sum(int(a[k, i]) << (32 * k) for k in range(a.shape[0])) for i in range(a.shape[1])]
        assert val(d) == val(ref), (lo, hi)
    gr = CE.backward(X, T, m, denom, torch.ones(1).cuda(), "sum")
    ref = oracle.ce_backward(x, t, rm, rd, np.ones(1, np.float32), "sum")
    assert np.array_equal(u32(gr), u32(ref))
