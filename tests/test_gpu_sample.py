"""GPU parity of the sampler (gr_sample) against the fp64 oracle, through the C ABI.

Every decision is an integer one (fixed-point weights, exact running sums), so the bar is
bit-exact: the tokens and the kept weights (Wk, Wp) of every row equal the oracle's.
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, say, torch_cuda

pytestmark = pytest.mark.gpu

# (temperature, top_p, top_k): greedy rows, nucleus only, top-k only, both, plain temperature
PARAM_MIX = [(0.0, 1.0, 0), (0.7, 0.9, 50), (1.0, 0.8, 0), (1.3, 1.0, 0), (0.5, 1.0, 7), (0.6, 0.95, 20),
             (1.0, 1.0, 1), (2.0, 0.5, 1000)]


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


@pytest.fixture(scope="module")
def gr():
    import continuous_quantized_decode_amd as gr
    gr.lib()
    return gr


def _run(gr, torch, logits, T, P, K, U):
    b = logits.shape[0]
    params = gr.sample_params(T, P, K, U, b=b)
    kept = torch.zeros((b, 2), dtype=torch.int64, device="cuda")
    tok = gr.gr_sample(dev(logits, torch), params, kept=kept)
    torch.cuda.synchronize()
    return host(tok), host(kept).view(np.uint64)


def _check(gr, torch, orc, logits, T, P, K, U, label):
    b = logits.shape[0]
    T, P, U = (np.broadcast_to(np.asarray(v, np.float64), (b,)).copy() for v in (T, P, U))
    K = np.broadcast_to(np.asarray(K, np.int32), (b,)).copy()
    say("sample", label, logits.shape)
    got, kept = _run(gr, torch, logits, T, P, K, U)
    want, wk, wp = orc.sample(logits, T, P, K, U, diag=True)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{label}: rows {bad[:8].tolist()} got {got[bad[:8]].tolist()} want {want[bad[:8]].tolist()}"
    np.testing.assert_array_equal(kept[:, 0], wk, err_msg=f"{label}: Wk")
    np.testing.assert_array_equal(kept[:, 1], wp, err_msg=f"{label}: Wp")
    return got


def _mix(b, rng):
    rows = [PARAM_MIX[i % len(PARAM_MIX)] for i in range(b)]
    T = np.array([r[0] for r in rows])
    P = np.array([r[1] for r in rows])
    K = np.array([r[2] for r in rows], np.int32)
    return T, P, K, synth.sample_uniforms(rng, b)


@pytest.mark.parametrize("vocab", [1, 5, 64, 4099, 32000, 128256, 151936])
def test_parameter_mix_bit_exact(torch, gr, orc, vocab):
    rng = np.random.default_rng(vocab)
    b = 16
    lg = synth.sample_logits(rng, b, vocab, spikes=min(8, vocab))
    _check(gr, torch, orc, lg, *_mix(b, rng), label=f"mix v={vocab}")


@pytest.mark.parametrize("seed", range(4))
def test_llama3_vocab_batch8_bit_exact(torch, gr, orc, seed):
    """The Llama-3-8B output head's vocabulary at batch 8, several draws per row."""
    rng = np.random.default_rng(1000 + seed)
    lg = synth.sample_logits(rng, 8, 128256, sigma=2.0 + seed)
    for rep in range(3):
        _check(gr, torch, orc, lg, *_mix(8, rng), label=f"llama3 seed={seed} rep={rep}")


@pytest.mark.parametrize("vocab", [4096, 4099])
def test_draws_on_running_weight_boundaries(torch, gr, orc, vocab):
    """u placed half a unit on either side of running-weight boundaries: any one-unit difference
    in a weight, or an off-by-one in the draw, changes the token."""
    rng = np.random.default_rng(77 + vocab)
    row = synth.sample_logits(rng, 1, vocab, sigma=1.5, spikes=4)[0]
    T = 0.9
    order = np.lexsort((np.arange(vocab), -row.astype(np.float64)))
    lmax = float(row[order[0]])
    w = np.array([orc.sample_weight((float(row[i]) - lmax) * (1.0 / T)) for i in order], np.uint64)
    cum = np.cumsum(w)
    total = float(cum[-1])
    js = np.unique(np.linspace(0, vocab - 2, 48).astype(int))
    js = js[w[js + 1] > 0]
    us = np.concatenate([(cum[js] - 0.5) / total, (cum[js] + 0.5) / total])
    lg = np.repeat(row[None], len(us), 0)
    got = _check(gr, torch, orc, lg, T, 1.0, 0, us, label=f"boundaries v={vocab}")
    np.testing.assert_array_equal(got[:len(js)], order[js])
    np.testing.assert_array_equal(got[len(js):], order[js + 1])


def test_degenerate_rows(torch, gr, orc):
    v = 1000
    rows, prm = [], []
    base = np.random.default_rng(5).normal(0, 2, v).astype(np.float32)

    def add(r, t=1.0, p=1.0, k=0, u=0.5):
        rows.append(np.asarray(r, np.float32))
        prm.append((t, p, k, u))

    add(np.full(v, 3.0), u=0.3217)                      # all equal: floor(u v)
    add(np.full(v, -np.inf), u=0.9)                     # all masked: index 0
    r = np.full(v, -np.inf); r[[17, 400, 999]] = [1.0, 2.0, 2.0]; add(r, u=0.7)
    r = base.copy(); r[::7] = np.nan; add(r, t=0.8, p=0.9, u=0.61)
    r = np.full(v, np.nan); add(r)                      # all NaN: index 0
    r = base.copy(); r[[3, 9]] = np.inf; add(r)         # infinite maximum: greedy
    r = base.copy(); r[:] = -1; r[[5, 2]] = [np.float32(-0.0), 0.0]; add(r, t=0.0)  # -0 == +0
    r = base.copy(); r[:] = -1; r[[5, 2]] = [np.float32(-0.0), 0.0]; add(r, t=1e-3, u=0.99)
    add(base, k=v - 1, u=0.999999)
    add(base, p=1e-9, u=0.8)                            # nucleus of one element
    add(base, p=0.0, u=0.8)
    add(base, t=1e-300, u=0.4)                          # huge 1/T: only the maximum weighs
    add(base, t=1e-320, u=0.4)                          # 1/T overflows: greedy
    add(base, t=np.inf, u=0.4321)                       # 1/T == 0: every finite logit weighs 2^31
    add(base, u=0.0)
    add(base, u=np.nextafter(1.0, 0.0))
    add(base, u=1.5)
    add(base, u=-2.0)
    add(base, t=np.nan)
    add(base, p=np.nan, k=-5, u=0.25)
    lg = np.stack(rows)
    T, P, K, U = (np.array([q[i] for q in prm]) for i in range(4))
    _check(gr, torch, orc, lg, T, P, K.astype(np.int32), U, label="degenerate")


@pytest.mark.parametrize("vocab", [128256, 4099])
def test_large_bins_take_the_row_pass_route(torch, gr, orc, vocab):
    """Rows whose level-1 bins exceed the LDS list: all-equal logits (the order is the index)
    and logits packed into a narrow band around 1."""
    rng = np.random.default_rng(31)
    b = 6
    lg = np.empty((b, vocab), np.float32)
    lg[:3] = 7.0
    lg[3:] = (1.0 + rng.normal(0, 1e-4, (3, vocab))).astype(np.float32)
    T = np.array([1.0, 0.5, 1.0, 1.0, 1e-4, 2e-5])
    P = np.array([1.0, 0.3, 0.9, 0.95, 1.0, 0.7])
    K = np.array([0, 0, 20000, 0, 9000, 0], np.int32)
    U = synth.sample_uniforms(rng, b)
    got = _check(gr, torch, orc, lg, T, P, K, U, label=f"large bins v={vocab}")
    assert got[0] == int(np.floor(U[0] * vocab))


def test_repeat_calls_reuse_the_workspace(torch, gr, orc):
    """The workspace carries nothing between calls: a second call with other rows and
    parameters on the same workspace matches the oracle."""
    rng = np.random.default_rng(8)
    ws = gr.workspace(gr.sample_workspace_size(8, 32000))
    for rep in range(2):
        lg = synth.sample_logits(rng, 8 - 3 * rep, 32000)
        T, P, K, U = _mix(8 - 3 * rep, rng)
        b = lg.shape[0]
        params = gr.sample_params(T, P, K, U, b=b)
        tok = host(gr.gr_sample(dev(lg, torch), params, ws=ws))
        np.testing.assert_array_equal(tok, orc.sample(lg, T, P, K, U))


@pytest.mark.parametrize("vocab", [128256, 4099])
def test_segments_with_few_and_many_candidates(torch, gr, orc, vocab):
    """Each 256-element segment holds 0 to 7 elements above a gap (the gathered prefix then
    mixes segments served from their top records with segments that must be read)."""
    rng = np.random.default_rng(55)
    b = 6
    lg = rng.normal(-4.0, 0.5, (b, vocab)).astype(np.float32)
    for r in range(b):
        for s0 in range(0, vocab, 256):
            m = (s0 // 256 + r) % 8
            idx = s0 + rng.choice(min(256, vocab - s0), min(m, vocab - s0), replace=False)
            lg[r, idx] = rng.uniform(2.0, 3.0, len(idx)).astype(np.float32)
    n_hi = int((lg[0] > 0).sum())
    T = np.array([0.5, 0.8, 1.0, 0.7, 1.2, 0.9])
    P = np.array([1.0, 0.9, 1.0, 0.5, 1.0, 0.99])
    K = np.array([n_hi, 0, n_hi // 2, 0, 0, 100], np.int32)
    U = synth.sample_uniforms(rng, b)
    _check(gr, torch, orc, lg, T, P, K, U, label=f"segment records v={vocab}")
