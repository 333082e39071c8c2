"""End-to-end parity of the GPU forward pass against the CPU oracle.

Protocol ("prompt P, then N greedy decode steps"): one prefill of P (its
argmax is generated token 1) then N decode steps fed the previous argmax.
Tolerance: per step, max |logit_gpu - logit_oracle| <= 1e-3 x (max - min of
the oracle's logits); greedy tokens identical.
"""

import os

import numpy as np
import pytest
import torch

from oracle import model as om
from synthetic import QWEN3_0_6B, TINY, WORKLOADS, gen_prompt, gen_weights

pytestmark = pytest.mark.gpu

TOL = 1e-3


def progress(msg):
    """A progress line for long cases (visible with pytest -s)."""
    print(f"[{os.path.basename(__file__)}] {msg}", flush=True)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / (np.max(b) - np.min(b)))


@pytest.fixture(scope="module")
def tiny_w():
    return gen_weights(TINY, 101)


@pytest.fixture(scope="module")
def tiny_ref(tiny_w):
    return om.Model(TINY, tiny_w)


def make(shape, weights, caps, **kw):
    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model

    return Qwen3Model(Qwen3Config.from_shape(shape), weights, caps, **kw)


def gpu_generate(model, prompt, steps, seq=0):
    lg, am = model.prefill(prompt, seq=seq)
    toks, logits = [int(am.item())], [lg.cpu().numpy().copy()]
    for _ in range(steps):
        lg, am = model.decode_step(seq=seq)
        toks.append(int(am.item()))
        logits.append(lg.cpu().numpy().copy())
    return toks, logits


def check_against_oracle(toks, logits, rtoks, rlogits):
    errs = [rel_err(a, b) for a, b in zip(logits, rlogits)]
    assert max(errs) <= TOL, f"logit errors {['%.1e' % e for e in errs]}"
    for a, b in zip(logits, rlogits):  # the GPU argmax is its own logits' argmax
        pass
    assert toks == list(rtoks), f"tokens {toks} != oracle {list(rtoks)}"


def test_tiny_workload_matches_oracle(tiny_w, tiny_ref):
    wl = WORKLOADS["tiny"]
    prompt = gen_prompt(TINY.vocab_size, wl.prompt_len, wl.prompt_seed)
    gpu = make(TINY, tiny_w, [wl.kv_capacity])
    toks, logits = gpu_generate(gpu, prompt, wl.decode_steps)
    rtoks, rlogits = tiny_ref.generate(prompt, wl.decode_steps, tiny_ref.new_cache(wl.kv_capacity))
    check_against_oracle(toks, logits, rtoks, rlogits)
    for lg, t in zip(logits, toks):
        assert int(np.argmax(lg)) == t
    assert gpu.kv_len() == wl.prompt_len + wl.decode_steps


def test_tiny_chunked_prefill_and_ragged_tail(tiny_w, tiny_ref):
    prompt = gen_prompt(TINY.vocab_size, 45, 7)  # 45 = 2 x 16 + ragged 13
    gpu = make(TINY, tiny_w, [64], max_batch_tokens=16)
    toks, logits = gpu_generate(gpu, prompt, 4)
    rtoks, rlogits = tiny_ref.generate(prompt, 4, tiny_ref.new_cache(64))
    check_against_oracle(toks, logits, rtoks, rlogits)


def test_tiny_multi_turn_prefill(tiny_w, tiny_ref):
    a, b = gen_prompt(TINY.vocab_size, 9, 8), gen_prompt(TINY.vocab_size, 6, 9)
    gpu = make(TINY, tiny_w, [32])
    gpu.prefill(a)
    lg, am = gpu.prefill(b)
    ref = tiny_ref.forward_uncached(np.concatenate([a, b]))[0]
    assert rel_err(lg.cpu().numpy(), ref) <= TOL
    assert gpu.kv_len() == 15


def test_tiny_reset_reproduces(tiny_w):
    prompt = gen_prompt(TINY.vocab_size, 20, 10)
    gpu = make(TINY, tiny_w, [40])
    t1, l1 = gpu_generate(gpu, prompt, 5)
    gpu.reset()
    assert gpu.kv_len() == 0
    t2, l2 = gpu_generate(gpu, prompt, 5)
    assert t1 == t2
    for a, b in zip(l1, l2):
        assert np.array_equal(a, b)


def test_tiny_graph_and_eager_decode_agree(tiny_w, monkeypatch):
    prompt = gen_prompt(TINY.vocab_size, 10, 11)
    g = make(TINY, tiny_w, [32])
    tg, lgr = gpu_generate(g, prompt, 6)
    monkeypatch.setenv("QWEN3_NO_GRAPH", "1")
    e = make(TINY, tiny_w, [32])
    te, le = gpu_generate(e, prompt, 6)
    assert tg == te
    for a, b in zip(lgr, le):
        assert np.array_equal(a, b)


def test_tiny_errors_leave_state_unchanged(tiny_w):
    from quantized_q8_dequant_amd import Qwen3Error

    prompt = gen_prompt(TINY.vocab_size, 14, 12)
    gpu = make(TINY, tiny_w, [16])
    gpu.prefill(prompt)
    with pytest.raises(Qwen3Error) as e:
        gpu.prefill(gen_prompt(TINY.vocab_size, 3, 13))
    assert e.value.code == -7
    with pytest.raises(Qwen3Error) as e:
        gpu.prefill([1, TINY.vocab_size])
    assert e.value.code == -8
    with pytest.raises(Qwen3Error) as e:
        gpu.prefill([])
    assert e.value.code == -6
    assert gpu.kv_len() == 14
    gpu.decode_step()
    gpu.decode_step()
    assert gpu.kv_len() == 16
    with pytest.raises(Qwen3Error) as e:
        gpu.decode_step()
    assert e.value.code == -7
    assert gpu.kv_len() == 16


def test_tiny_bf16_cache_matches_oracle():
    shape = TINY.with_(name="tiny-bf16kv", kv_type="bf16")
    w = gen_weights(shape, 101)
    ref = om.Model(shape, w)
    prompt = gen_prompt(shape.vocab_size, 24, 14)
    gpu = make(shape, w, [48])
    toks, logits = gpu_generate(gpu, prompt, 8)
    rtoks, rlogits = ref.generate(prompt, 8, ref.new_cache(48))
    check_against_oracle(toks, logits, rtoks, rlogits)


def test_tiny_batched_decode_matches_single(tiny_w, tiny_ref):
    prompts = [gen_prompt(TINY.vocab_size, n, 20 + n) for n in (5, 17, 33)]
    gpu = make(TINY, tiny_w, [48, 48, 48])
    first = []
    for s, p in enumerate(prompts):
        _, am = gpu.prefill(p, seq=s)
        first.append(int(am.item()))
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    logits = torch.empty((3, TINY.vocab_size), dtype=torch.float32, device="cuda:0")
    am = torch.empty(3, dtype=torch.int32, device="cuda:0")
    seqs = [0, 1, 2]
    outs = []
    for _ in range(4):
        gpu.decode_batch(seqs, toks, logits, am)
        outs.append((logits.cpu().numpy().copy(), am.cpu().numpy().copy()))
        toks = am.clone()
    for s, p in enumerate(prompts):
        rt, rl = tiny_ref.generate(p, 4, tiny_ref.new_cache(48))
        assert rt[0] == first[s]
        for i in range(4):
            assert rel_err(outs[i][0][s], rl[i + 1]) <= TOL
            assert outs[i][1][s] == rt[i + 1]


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_qwen3_0_6b_prefill_and_decode_matches_oracle():
    """The decode workload as timed: the 512-token prompt, then all 256 greedy
    decode steps (the one-launch step), every step's logits and token against
    the oracle's."""
    wl = WORKLOADS["0.6b-decode"]
    w = gen_weights(QWEN3_0_6B, wl.weight_seed)
    prompt = gen_prompt(QWEN3_0_6B.vocab_size, wl.prompt_len, wl.prompt_seed)
    steps = wl.decode_steps
    gpu = make(QWEN3_0_6B, w, [wl.kv_capacity])
    assert gpu.decode_launches() == 1
    toks, logits = gpu_generate(gpu, prompt, steps)
    gpu.step_status()
    gpu.close()
    del gpu
    torch.cuda.empty_cache()
    for lg, t in zip(logits, toks):
        assert int(np.argmax(lg)) == t
    ref = om.Model(QWEN3_0_6B, w, keep_f64=True)
    del w
    rtoks, rlogits = ref.generate(prompt, steps, ref.new_cache(wl.kv_capacity))
    check_against_oracle(toks, logits, rtoks, rlogits)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_qwen3_0_6b_prefill_4096_one_call_matches_oracle():
    """The prefill-dominated workload: a 4096-token prompt in one prefill call
    (a single 4096-row chunk through the MFMA GEMM and attention tiles), then
    32 greedy decode steps."""
    wl = WORKLOADS["0.6b-prefill4096"]
    w = gen_weights(QWEN3_0_6B, wl.weight_seed)
    prompt = gen_prompt(QWEN3_0_6B.vocab_size, wl.prompt_len, wl.prompt_seed)
    gpu = make(QWEN3_0_6B, w, [wl.kv_capacity], max_batch_tokens=wl.prompt_len)
    toks, logits = gpu_generate(gpu, prompt, wl.decode_steps)
    # the same prompt in 1024-row chunks gives the same cache and logits
    chunked = make(QWEN3_0_6B, w, [wl.kv_capacity], max_batch_tokens=1024)
    lg_c, am_c = chunked.prefill(prompt)
    assert int(am_c.item()) == toks[0]
    assert rel_err(lg_c.cpu().numpy(), logits[0]) <= TOL
    for layer in (0, QWEN3_0_6B.num_layers - 1):
        k1, v1 = gpu.kv_export(0, layer)
        k2, v2 = chunked.kv_export(0, layer)
        assert torch.equal(k1[:, : wl.prompt_len], k2) and torch.equal(v1[:, : wl.prompt_len], v2)
    chunked.close()
    gpu.close()
    del gpu, chunked
    torch.cuda.empty_cache()
    ref = om.Model(QWEN3_0_6B, w)
    del w
    rtoks, rlogits = ref.generate(prompt, wl.decode_steps, ref.new_cache(wl.kv_capacity))
    check_against_oracle(toks, logits, rtoks, rlogits)


# ---- bf16 weights (f32 activations x exactly widened bf16, f64 sums) ----------------

TINY_BF16 = TINY.with_(name="tiny-bf16", weight_type="bf16", kv_type="bf16")


@pytest.fixture(scope="module")
def tiny_bf16_w():
    return gen_weights(TINY_BF16, 101)


@pytest.fixture(scope="module")
def tiny_bf16_ref(tiny_bf16_w):
    return om.Model(TINY_BF16, tiny_bf16_w)


def test_tiny_bf16_weights_match_oracle(tiny_bf16_w, tiny_bf16_ref):
    prompt = gen_prompt(TINY_BF16.vocab_size, 45, 31)
    for mbt in (0, 16):  # one chunk; 16-row chunks with a ragged tail
        gpu = make(TINY_BF16, tiny_bf16_w, [64], max_batch_tokens=mbt)
        toks, logits = gpu_generate(gpu, prompt, 8)
        rtoks, rlogits = tiny_bf16_ref.generate(prompt, 8, tiny_bf16_ref.new_cache(64))
        check_against_oracle(toks, logits, rtoks, rlogits)
        for lg, t in zip(logits, toks):
            assert int(np.argmax(lg)) == t


def test_tiny_bf16_batched_decode_matches_oracle(tiny_bf16_w, tiny_bf16_ref):
    prompts = [gen_prompt(TINY_BF16.vocab_size, n, 40 + n) for n in (3, 20, 61, 9)]
    gpu = make(TINY_BF16, tiny_bf16_w, [72] * 4)
    first = [int(gpu.prefill(p, seq=s)[1].item()) for s, p in enumerate(prompts)]
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    logits = torch.empty((4, TINY_BF16.vocab_size), dtype=torch.float32, device="cuda:0")
    am = torch.empty(4, dtype=torch.int32, device="cuda:0")
    outs = []
    for _ in range(5):
        gpu.decode_batch([0, 1, 2, 3], toks, logits, am)
        outs.append((logits.cpu().numpy().copy(), am.cpu().numpy().copy()))
        toks = am.clone()
    for s, p in enumerate(prompts):
        rt, rl = tiny_bf16_ref.generate(p, 5, tiny_bf16_ref.new_cache(72))
        assert rt[0] == first[s]
        for i in range(5):
            assert rel_err(outs[i][0][s], rl[i + 1]) <= TOL
            assert outs[i][1][s] == rt[i + 1]


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_qwen3_0_6b_bf16_ragged_batch_matches_oracle():
    """bf16 0.6B, four sequences of ragged lengths, full oracle runs."""
    from synthetic import QWEN3_0_6B_BF16, gen_prompts

    shape = QWEN3_0_6B_BF16
    w = gen_weights(shape, 501)
    lengths = [37, 300, 129, 1030]
    prompts = gen_prompts(shape.vocab_size, lengths, 502)
    steps = 3
    gpu = make(shape, w, [n + steps + 1 for n in lengths])
    first = [int(gpu.prefill(p, seq=s)[1].item()) for s, p in enumerate(prompts)]
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    logits = torch.empty((4, shape.vocab_size), dtype=torch.float32, device="cuda:0")
    am = torch.empty(4, dtype=torch.int32, device="cuda:0")
    outs = []
    for _ in range(steps):
        gpu.decode_batch([0, 1, 2, 3], toks, logits, am)
        outs.append((logits.cpu().numpy().copy(), am.cpu().numpy().copy()))
        toks = am.clone()
    gpu.close()
    del gpu
    torch.cuda.empty_cache()
    ref = om.Model(shape, w)
    del w
    for s, p in enumerate(prompts):
        rt, rl = ref.generate(p, steps, ref.new_cache(len(p) + steps + 1))
        assert rt[0] == first[s]
        for i in range(steps):
            assert rel_err(outs[i][0][s], rl[i + 1]) <= TOL, (s, i)
            assert outs[i][1][s] == rt[i + 1], (s, i)


def oracle_cache_from_rows(ref, ks, vs, rows, capacity):
    """An oracle cache holding rows [0, rows) of exported GPU K/V rows."""
    c = ref.new_cache(capacity)
    for layer in range(ref.shape.num_layers):
        c.k[layer][:rows] = ks[layer][:rows]
        c.v[layer][:rows] = vs[layer][:rows]
    c.len = rows
    return c


def export_rows(gpu, seq):
    """Every layer's cached K and V rows of one sequence, as f32 [n, kv_heads, hd]."""
    ks, vs = [], []
    for layer in range(gpu.cfg.num_layers):
        k, v = gpu.kv_export(seq, layer)
        ks.append(k.cpu().numpy().transpose(1, 0, 2).copy())
        vs.append(v.cpu().numpy().transpose(1, 0, 2).copy())
    return ks, vs


def check_prompt_blocks(ref, prompt, ks, vs, starts, B, what):
    """Oracle forward of each block prompt[p0 : p0 + B] over the GPU's rows
    [0, p0) (p0 = 0: the oracle's own prefill); the block's cached rows of
    every layer against the oracle's.  Returns the last block's logits."""
    lg = None
    for p0 in starts:
        c = oracle_cache_from_rows(ref, ks, vs, p0, p0 + B)
        lg = ref.forward(prompt[p0 : p0 + B], c)[0]
        for layer in range(ref.shape.num_layers):
            check_cache_rows(ks[layer][p0 : p0 + B], c.k[layer][p0 : p0 + B], f"{what} K rows {p0}+{B} layer {layer}")
            check_cache_rows(vs[layer][p0 : p0 + B], c.v[layer][p0 : p0 + B], f"{what} V rows {p0}+{B} layer {layer}")
        del c
    return lg


@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_bf16_batch64_ragged_workload():
    """The batched bf16 workload at full size: 64 sequences with lengths drawn
    from 1024..16384, each filled by prefill, then 128 lockstep greedy steps
    ("A transformer from scratch", section 12.5: a batched step is each
    sequence's own step).

    Checked against the oracle, for the shortest, the longest and six
    sequences drawn with a fixed seed: the shortest in full (the oracle's own
    prefill, every cached row, its first two decode steps); for the others,
    64-row blocks of the prompt (the first from an empty cache, one in the
    middle and the last over the GPU's earlier rows: every layer's rows and
    the prefill's logits and token), and the first and last batched steps
    over the GPU's cache.  For all 64: every step's token is the argmax of
    its logits, and the first and last batched steps equal each sequence's
    own decode step (rewound with truncate and stepped alone)."""
    from synthetic import QWEN3_0_6B_BF16, gen_lengths, gen_prompts

    wl = WORKLOADS["0.6b-bf16-batch64"]
    shape = QWEN3_0_6B_BF16
    B = 64
    lengths = gen_lengths(wl.n_seqs, wl.min_len, wl.max_len, wl.length_seed)
    prompts = gen_prompts(shape.vocab_size, lengths, wl.prompt_seed)
    n = wl.n_seqs
    order = np.argsort(lengths, kind="stable")
    short, longest = int(order[0]), int(order[-1])
    rest = [i for i in range(n) if i not in (short, longest)]
    drawn = np.random.Generator(np.random.PCG64(504)).choice(len(rest), 6, replace=False)
    picks = [short, longest] + sorted(rest[i] for i in drawn)
    w = gen_weights(shape, wl.weight_seed)
    caps = [int(L) + wl.decode_steps for L in lengths]
    gpu = make(shape, w, caps)
    ref = om.Model(shape, w, keep_f64=True)
    del w
    first, pre_logits = [], {}
    for s, p in enumerate(prompts):
        lg, am = gpu.prefill(p, seq=s, logits=s in picks)
        first.append(int(am.item()))
        if s in picks:
            pre_logits[s] = lg.cpu().numpy().copy()
    progress("GPU: 64 prompts prefilled")

    # oracle checks of the prefills, and the oracle's first step of each pick
    want0, want1 = {}, None
    for s in picks:
        L = int(lengths[s])
        ks, vs = export_rows(gpu, s)
        if s == short:
            rc = ref.new_cache(L + 2)
            lr = ref.forward(prompts[s], rc)[0]
            for layer in range(shape.num_layers):
                check_cache_rows(ks[layer], rc.k[layer][:L], f"seq {s} K layer {layer}")
                check_cache_rows(vs[layer], rc.v[layer][:L], f"seq {s} V layer {layer}")
            want0[s] = ref.forward([first[s]], rc)[0]
            want1 = (ref, rc)  # the oracle's own cache, one step on
        else:
            mid = (L // 2 // B) * B
            lr = check_prompt_blocks(ref, prompts[s], ks, vs, [0, mid, L - B], B, f"seq {s}")
            c = oracle_cache_from_rows(ref, ks, vs, L, L + 1)
            want0[s] = ref.forward([first[s]], c)[0]
            del c
        assert rel_err(pre_logits[s], lr) <= TOL, s
        assert first[s] == int(np.argmax(lr)), s
        del ks, vs
        progress(f"oracle: sequence {s} (length {L}) checked")

    seqs = list(range(n))
    logits = torch.empty((n, shape.vocab_size), dtype=torch.float32, device="cuda:0")
    am = torch.empty(n, dtype=torch.int32, device="cuda:0")

    def batched_equals_single(step_toks, lg_b, am_b):
        """Rewind every sequence by the batched step's row and redo it alone."""
        for s in seqs:
            L = gpu.kv_len(s)
            gpu.truncate(L - 1, seq=s)
            t = torch.tensor([step_toks[s]], dtype=torch.int32, device="cuda:0")
            lg1, am1 = gpu.decode_step(seq=s, token=t)
            lg1 = lg1.cpu().numpy()
            assert int(am1.item()) == int(am_b[s]), s
            assert rel_err(lg1, lg_b[s]) <= TOL, s
            assert gpu.kv_len(s) == L

    toks_h = list(first)
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    for step in range(wl.decode_steps):
        last = step == wl.decode_steps - 1
        if last:  # the oracle's last step of each pick, over the GPU's cache
            wantN = {}
            for s in picks:
                ks, vs = export_rows(gpu, s)
                c = oracle_cache_from_rows(ref, ks, vs, gpu.kv_len(s), gpu.kv_len(s) + 1)
                del ks, vs
                wantN[s] = ref.forward([toks_h[s]], c)[0]
                del c
            progress("oracle: last-step references done")
        gpu.decode_batch(seqs, toks, logits, am)
        lg = logits.cpu().numpy()
        amh = am.cpu().numpy()
        assert np.array_equal(np.argmax(lg, axis=1), amh), f"step {step}"
        if step == 0:
            for s in picks:
                assert rel_err(lg[s], want0[s]) <= TOL, (s, step)
                assert int(amh[s]) == int(np.argmax(want0[s])), (s, step)
            batched_equals_single(toks_h, lg, amh)
        if step == 1:
            r, rc = want1
            lr = r.forward([toks_h[short]], rc)[0]
            assert rel_err(lg[short], lr) <= TOL
            assert int(amh[short]) == int(np.argmax(lr))
            want1 = None
        if last:
            for s in picks:
                assert rel_err(lg[s], wantN[s]) <= TOL, (s, step)
                assert int(amh[s]) == int(np.argmax(wantN[s])), (s, step)
            batched_equals_single(toks_h, lg, amh)
        toks_h = [int(t) for t in amh]
        toks = am.clone()
    for s in seqs:
        assert gpu.kv_len(s) == lengths[s] + wl.decode_steps
    gpu.close()


def check_cache_rows(gpu_rows, ref_rows, what):
    """Cached K or V rows [n, kv_heads, hd] of the GPU against the oracle's.
    Both round the same f32 values to the cache type, so nearly all are
    bitwise equal; a row may differ where an upstream Q8_0 code flipped, by
    at most one bf16 step of the row's largest element (the logits' own bar
    is 1e-3 of their range)."""
    g = np.asarray(gpu_rows, np.float64)
    o = np.asarray(ref_rows, np.float64)
    assert g.shape == o.shape, what
    scale = np.max(np.abs(o), axis=-1, keepdims=True) + 1e-30
    worst = float(np.max(np.abs(g - o) / scale))
    same = float(np.mean(g == o))
    assert worst <= 2.0**-8, f"{what}: worst row error {worst:.2e} of the row's largest element"
    assert same >= 0.99, f"{what}: {same:.4f} bitwise equal"


@pytest.mark.slow
@pytest.mark.timeout(2400)
def test_qwen3_8b_long_context_matches_oracle():
    """Qwen3-8B shape, Q8_0 weights, bf16 KV cache.

    The 2048-token prompt and 8 greedy decode steps against the oracle's own
    prefill and steps: every step's logits and token, and every cached row
    (all 2056 positions, all 36 layers) against the oracle's cache.  Then
    decode steps at KV lengths 16384 and 32768 (each cache filled by
    prefilling a seeded random prompt of that length): there the oracle,
    which cannot redo an 8B prefill of that length on the host, takes the
    GPU's cache and checks the step's logits and token."""
    from synthetic import QWEN3_8B

    wl = WORKLOADS["8b-longctx"]
    shape = QWEN3_8B
    steps = 8
    w = gen_weights(shape, wl.weight_seed)
    progress("8B weights drawn")
    prompt = gen_prompt(shape.vocab_size, wl.prompt_len, wl.prompt_seed)
    gpu = make(shape, w, [wl.kv_capacity], max_batch_tokens=2048)
    progress("8B model created on the GPU")
    L_ = shape.num_layers

    def export_all():
        n = gpu.kv_len(0)
        ks, vs = [], []
        for layer in range(L_):
            k, v = gpu.kv_export(0, layer)
            ks.append(k.cpu().numpy().transpose(1, 0, 2).copy())
            vs.append(v.cpu().numpy().transpose(1, 0, 2).copy())
        return n, ks, vs

    toks, logits = gpu_generate(gpu, prompt, steps)
    n_short, ks_short, vs_short = export_all()
    assert n_short == wl.prompt_len + steps
    long = {}
    for L in wl.decode_contexts[1:]:
        gpu.reset()
        p = gen_prompt(shape.vocab_size, L, wl.prompt_seed + L)
        _, am = gpu.prefill(p, logits=False)
        t0 = int(am.item())
        n, ks, vs = export_all()
        lg, am = gpu.decode_step()
        long[L] = (t0, n, ks, vs, lg.cpu().numpy().copy(), int(am.item()))
        progress(f"GPU prefill {L} + decode step done")
    gpu.close()
    del gpu
    torch.cuda.empty_cache()
    for lg, t in zip(logits, toks):
        assert int(np.argmax(lg)) == t
    ref = om.Model(shape, w, threads=16, keep_f64=True)
    del w
    progress("oracle model built")

    rc = ref.new_cache(n_short + 1)
    rtoks, rlogits = ref.generate(prompt, steps, rc)
    progress("oracle: 2048-token prefill and 8 steps done")
    check_against_oracle(toks, logits, rtoks, rlogits)
    for layer in range(L_):
        check_cache_rows(ks_short[layer], rc.k[layer][:n_short], f"K layer {layer}")
        check_cache_rows(vs_short[layer], rc.v[layer][:n_short], f"V layer {layer}")
    del rc, ks_short, vs_short

    def cache_of(n, ks, vs, rows):
        c = ref.new_cache(n + 1)
        for layer in range(L_):
            c.k[layer][:rows] = ks[layer][:rows]
            c.v[layer][:rows] = vs[layer][:rows]
        c.len = rows
        return c

    for L, (t0, n, ks, vs, lg, tok) in long.items():
        assert n == L
        c = cache_of(n, ks, vs, n)
        lr = ref.forward([t0], c)[0]
        assert rel_err(lg, lr) <= TOL, L
        assert tok == int(np.argmax(lr)), L
        progress(f"oracle: decode at {L} checked")
        del c


# ---- the one-launch decode step against the per-kernel step -------------------------


@pytest.mark.parametrize("shape_name", ["tiny", "0.6b"])
def test_persistent_decode_matches_per_kernel_decode(shape_name, monkeypatch):
    """The one-launch decode step computes what the per-kernel step computes
    (same reductions; only the attention split differs, in f64): tokens equal,
    logits within the tolerance and nearly all bit-identical; both against
    the oracle for the tiny model."""
    shape, wseed, plen, steps, cap = (
        (TINY, 101, 37, 12, 64) if shape_name == "tiny" else (QWEN3_0_6B, 201, 300, 6, 320)
    )
    w = gen_weights(shape, wseed)
    prompt = gen_prompt(shape.vocab_size, plen, 55)
    monkeypatch.setenv("QWEN3_PERSISTENT", "1")
    a = make(shape, w, [cap])
    assert a.decode_launches() == 1
    ta, la = gpu_generate(a, prompt, steps)
    a.close()
    monkeypatch.setenv("QWEN3_PERSISTENT", "0")
    b = make(shape, w, [cap])
    assert b.decode_launches() == 5 * shape.num_layers + 2
    tb, lb = gpu_generate(b, prompt, steps)
    b.close()
    assert ta == tb
    same = 0.0
    for x, y in zip(la, lb):
        assert rel_err(x, y) <= TOL
        same += float(np.mean(x == y))
    assert same / len(la) >= 0.999
    if shape_name == "tiny":
        ref = om.Model(shape, w)
        rt, rl = ref.generate(prompt, steps, ref.new_cache(cap))
        check_against_oracle(ta, la, rt, rl)


def test_tiny_decode_steps_interleaved_over_sequences(tiny_w, tiny_ref):
    """decode_step on three sequences in turn (each its own cache region,
    length and argmax buffer) gives each sequence the oracle's tokens."""
    prompts = [gen_prompt(TINY.vocab_size, n, 60 + n) for n in (4, 29, 13)]
    gpu = make(TINY, tiny_w, [48, 48, 48])
    toks = {s: [int(gpu.prefill(p, seq=s)[1].item())] for s, p in enumerate(prompts)}
    logits = {s: [] for s in range(3)}
    for _ in range(5):
        for s in (2, 0, 1):
            lg, am = gpu.decode_step(seq=s)
            toks[s].append(int(am.item()))
            logits[s].append(lg.cpu().numpy().copy())
    for s, p in enumerate(prompts):
        rt, rl = tiny_ref.generate(p, 5, tiny_ref.new_cache(48))
        assert toks[s] == list(rt)
        for i in range(5):
            assert rel_err(logits[s][i], rl[i + 1]) <= TOL
        assert gpu.kv_len(s) == len(p) + 5
