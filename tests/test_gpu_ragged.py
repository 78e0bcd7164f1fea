"""GPU parity of ragged serving batches: masked decode and spec steps, per-slot loads.

Sequences of a serving batch join and leave at their own times ([DE]
"ReplaySSM beschleunigt ...", section "Warum es wichtig ist": the gain comes
from many concurrent sequences; [TR] "NVIDIA ve Dao AI Lab ...", section
"ReplaySSM nasil calisir?": every sequence flushes its own 16-entry buffer).
Checked through the C ABI against the oracle:
  * the hand-derived bookkeeping traces of tests/golden (masked steps, arrivals,
    staggered windows) reproduced bit for bit by the GPU;
  * masked decode / spec / commit and per-slot loads at small shapes, every
    checkpoint dtype and with read copies: outputs of the active sequences,
    checkpoints and bookkeeping as for the other parity tests, and the output
    rows of the sequences left out untouched;
  * the same in a layer stack (one mask for every layer of a step);
  * the batch-256 Mamba-2 and GDN layers with a seeded occupancy pattern
    (sequences leaving and arriving mid-window), sampled sequences against the
    oracle;
  * host-side validation of the new entry points.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from hybrid_decode_replay_amd import synth  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_decode_replay_amd import binding  # noqa: F401  (fails loudly if not built)
    yield


def rb():
    from hybrid_decode_replay_amd import binding
    return binding


def _toks(kind, seed, T, B, H, G, C, R, io="f32"):
    if kind == "mamba2":
        return synth.mamba2_tokens(seed, T, B, H, G, C, R, dtype=io)
    return synth.gdn_tokens(seed, T, B, H, G, R, C, dtype=io)


def _golden(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                tok = line.split()
                out.append((tok[0], tok[1], list(map(int, tok[2:]))))
    return out


def _mask(s):
    return np.array([c == "1" for c in s])


@pytest.mark.parametrize("name,stagger", [("bookkeeping_ragged_cap4.txt", False),
                                          ("bookkeeping_stagger_slots_cap4.txt", True)])
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_golden_trace_on_gpu(kind, name, stagger):
    """The GPU's bookkeeping after every operation equals the hand-derived trace; values
    are checked against the oracle along the way (harness.Pair)."""
    from harness import Pair
    b = rb()
    B, H, C, R, cap = 3, 2, 32, 32, 4
    G = 1 if kind == "mamba2" else H
    pair = Pair(b.MAMBA2 if kind == "mamba2" else b.GDN, B, H, G, C, R, cap=cap, io=b.F32, seed=81,
                S0=synth.checkpoint(81, (B, H, C, R)), flags=b.FLAG_STAGGER_FLUSH if stagger else 0)
    toks = _toks(kind, 81, 64, B, H, G, C, R)
    t = 0
    for i, (op, arg, want) in enumerate(_golden(name)):
        what = f"line {i}: {op} {arg}"
        if op == "decode":
            pair.decode(synth.token(toks, t), what=what, active=_mask(arg)); t += 1
        elif op == "spec":
            k, m = arg.split(":")
            pair.spec({n: v[t:t + int(k)] for n, v in toks.items()}, what=what, active=_mask(m)); t += int(k)
        elif op == "commit":
            pair.commit([int(a) for a in arg.split(",")], what=what)
        elif op == "load":
            slots = [int(a) for a in arg.split(",")]
            pair.load_slots(slots, synth.checkpoint(82 + i, (len(slots), H, C, R)), what=what)
        elif op == "flush":
            pair.flush(what=what)
        L, Pd, F, E = pair.st.read_book()
        got = L.tolist() + Pd.tolist() + F.tolist() + [int(E[0])]
        assert got == want, (what, got, want)


CASES = [("f32", None, "f32"), ("bf16", None, "f32"), ("f32", "fp8", "f32"), ("bf16", "mxfp4", "f32"),
         ("f32", None, "f16"), ("f32", None, "fp8"), ("f32", "mxfp4", "fp8")]


@pytest.mark.parametrize("io,rc,ck", CASES)
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_masked_steps_and_arrivals(kind, io, rc, ck):
    from harness import Pair
    b = rb()
    B, H, C, R, cap = 6, 2, 48, 64, 5
    G = 1 if kind == "mamba2" else H
    pair = Pair(b.MAMBA2 if kind == "mamba2" else b.GDN, B, H, G, C, R, cap=cap,
                io=b.BF16 if io == "bf16" else b.F32, seed=83, S0=synth.checkpoint(83, (B, H, C, R), std=0.5),
                read_copy={None: b.NONE, "fp8": b.FP8_E4M3, "mxfp4": b.MXFP4}[rc],
                ckpt={"f32": b.F32, "f16": b.F16, "fp8": b.FP8_E4M3}[ck])
    toks = _toks(kind, 83, 120, B, H, G, C, R, io)
    rng = np.random.default_rng(83)
    t = 0
    print(f"[ragged] {kind} io={io} copy={rc} ckpt={ck}", flush=True)
    for step in range(30):
        r = rng.random()
        active = rng.random(B) < 0.7
        if r < 0.55:
            y = pair.decode(synth.token(toks, t), what=f"step {step} decode", active=active); t += 1
            torch.cuda.synchronize()
            # rows of sequences that sat out were never written (the binding starts y at zero)
            assert not y[0, torch.from_numpy(~active).cuda()].float().abs().sum().item(), step
        elif r < 0.8:
            k = int(rng.integers(1, cap + 1))
            y = pair.spec({n: v[t:t + k] for n, v in toks.items()}, what=f"step {step} spec {k}", active=active)
            t += k
            torch.cuda.synchronize()
            assert not y[:, torch.from_numpy(~active).cuda()].float().abs().sum().item(), step
            acc = np.where(active, rng.integers(0, k + 1, size=B), 0)
            if rng.random() < 0.3:
                pair.rollback(what=f"step {step} rollback")
            else:
                pair.commit(acc, what=f"step {step} commit")
        elif r < 0.9:
            n = int(rng.integers(1, 3))
            slots = sorted(rng.choice(B, size=n, replace=False).tolist())
            pair.load_slots(slots, synth.checkpoint(84 + step, (n, H, C, R), std=0.5), what=f"step {step} arrive")
        else:
            pair.flush(what=f"step {step} flush")
    print("max errors", pair.max_err, flush=True)


def test_stack_masked_and_arrivals():
    """A two-layer stack (Mamba-2 + GDN): masked steps with one mask for both layers, a
    per-slot arrival in every layer, a masked spec round with commit."""
    from harness import Pair, check_book
    from oracle import replay_oracle as ro
    b = rb()
    B, cap = 5, 4
    pm = Pair(b.MAMBA2, B, 2, 1, 32, 64, cap=cap, io=b.F32, seed=85, S0=synth.checkpoint(85, (B, 2, 32, 64)))
    pg = Pair(b.GDN, B, 2, 2, 32, 64, cap=cap, io=b.F32, seed=86, S0=synth.checkpoint(86, (B, 2, 32, 64)),
              read_copy=b.FP8_E4M3)
    pairs = [pm, pg]
    toks = [synth.mamba2_tokens(85, 40, B, 2, 1, 32, 64), synth.gdn_tokens(86, 40, B, 2, 2, 64, 32)]
    stk = b.ReplayStack([p.st for p in pairs])
    so = ro.StackSession([p.orc for p in pairs])
    rng = np.random.default_rng(85)
    t = 0
    for step in range(10):
        active = rng.random(B) < 0.6
        act = torch.from_numpy(active.astype(np.uint8)).cuda()
        for l, p in enumerate(pairs):
            tok = synth.token(toks[l], t)
            y = stk.decode_layer(l, p.to_dev(tok), p.params, active=act)
            yo = so.decode_layer(l, tok, active=active)
            sel = np.flatnonzero(active)
            if sel.size:
                p.check_outputs(y[:, sel.tolist()], yo[None][:, sel], f"step {step} layer {l}")
        t += 1
        for l, p in enumerate(pairs):
            p.check_ckpt(f"step {step} layer {l}")
        check_book(stk.read_book(), so, f"step {step}")
        if step == 4:
            S = [synth.checkpoint(87 + l, (2,) + p.st.ckpt_shape[1:]) for l, p in enumerate(pairs)]
            stk.load_slots([4, 0], [torch.from_numpy(s).cuda() for s in S])
            so.load_slots([4, 0], S)
            for l, p in enumerate(pairs):
                p.check_ckpt(f"arrival layer {l}")
            check_book(stk.read_book(), so, "arrival")
    active = np.array([1, 0, 1, 1, 0], bool)
    act = torch.from_numpy(active.astype(np.uint8)).cuda()
    for l, p in enumerate(pairs):
        drafts = {n: v[t:t + 3] for n, v in toks[l].items()}
        y = stk.spec_layer(l, 3, p.to_dev(drafts), p.params, active=act)
        yo = np.stack(so.spec_layer(l, [synth.token(toks[l], t + j) for j in range(3)], active=active))
        sel = np.flatnonzero(active)
        p.check_outputs(y[:, sel.tolist()], yo[:, sel], f"spec layer {l}")
    acc = [2, 0, 3, 1, 0]
    stk.commit(torch.tensor(acc, dtype=torch.int32, device="cuda"))
    so.commit(acc)
    for l, p in enumerate(pairs):
        p.check_ckpt(f"commit layer {l}")
    check_book(stk.read_book(), so, "commit")
    # one mask per step: a different mask pointer for the second layer is refused
    other = act.clone()
    stk.decode_layer(0, pm.to_dev(synth.token(toks[0], t + 3)), pm.params, active=act)
    with pytest.raises(b.ReplayError) as e:
        stk.decode_layer(1, pg.to_dev(synth.token(toks[1], t + 3)), pg.params, active=other)
    assert e.value.status == b.ERR_STATE


def test_host_validation_of_ragged_entry_points():
    import ctypes
    b = rb()
    B, H, C, R = 4, 2, 32, 32
    st = b.ReplayState(b.make_config(b.MAMBA2, B, H, 1, C, R, 4, b.F32))
    S = torch.zeros((2, H, C, R), device="cuda")

    def status(slots, n=None, ptr=S):
        arr = (ctypes.c_int32 * len(slots))(*slots)
        return b.lib().replay_load_slots(st.h, len(slots) if n is None else n, arr,
                                          ctypes.c_void_p(ptr.data_ptr()), None)

    assert status([0, 0]) == b.ERR_ARG             # a slot twice
    assert status([0, 4]) == b.ERR_ARG             # out of range
    assert status([-1, 2]) == b.ERR_ARG
    assert status([0, 1], n=0) == b.ERR_ARG
    assert status([0, 1], n=5) == b.ERR_ARG
    assert status([2, 3]) == b.OK
    A, D = synth.mamba2_params(0, H)
    params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
    tok = {k: torch.from_numpy(v).cuda() for k, v in synth.token(synth.mamba2_tokens(0, 2, B, H, 1, C, R), 0).items()}
    ri = b.make_inputs(st.cfg, tok, params)
    y = torch.empty((1, B, H, C), device="cuda")
    assert b.lib().replay_decode_step_masked(st.h, ctypes.byref(ri), None, ctypes.c_void_p(y.data_ptr()),
                                             None) == b.ERR_ARG
    drafts = {k: v[None] for k, v in tok.items()}
    act = torch.ones(B, dtype=torch.uint8, device="cuda")
    st.spec_append(1, drafts, params, active=act)
    assert status([0, 1]) == b.ERR_STATE           # drafts pending
    st.rollback()
    torch.cuda.synchronize()
    # a state bound to a stack cannot be freed before the stack
    st2 = b.ReplayState(b.make_config(b.MAMBA2, B, H, 1, C, R, 4, b.F32))
    stk = b.ReplayStack([st, st2])
    assert b.lib().replay_state_free(st2.h) == b.ERR_STATE
    stk.free()
    assert b.lib().replay_state_free(st2.h) == b.OK
    st2.h = None


def test_fp32_load_rounding_planted_values():
    """replay_load_checkpoint_f32 rounds on the device with the library's encoders: codes equal
    the oracle's E4M3 encoder (saturating at 448, NaN to 0x7f) and binary16 round to nearest
    even (overflow to inf) on values placed at every edge."""
    from oracle import replay_oracle as ro
    b = rb()
    edges = [0.0, -0.0, 448.0, 449.0, 463.9, 464.0, 464.1, 500.0, 1e6, -1e6, np.inf, -np.inf, 2.0 ** -9,
             2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6, 240.0, 248.0, 0.5 + 2.0 ** -5, 1.0625, 1.1875, -448.5,
             65504.0, 65519.99, 65520.0, 70000.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14,
             1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2049.0, 2051.0, 1e-30, -3.0e-8]
    B, H, C, R = 2, 1, 16, 32
    vals = np.resize(np.array(edges, np.float32), B * H * C * R).reshape(B, H, C, R)
    rng = np.random.default_rng(0)
    vals = vals * np.where(rng.random(vals.shape) < 0.3, -1.0, 1.0).astype(np.float32)
    vals[0, 0, 0, :3] = [np.nan, -np.nan, 1.0]
    for ck in (b.FP8_E4M3, b.F16):
        st = b.ReplayState(b.make_config(b.MAMBA2, B, H, 1, C, R, 4, b.F32, ckpt_dtype=ck))
        st.load_checkpoint(torch.from_numpy(vals).cuda())
        back = st.read_checkpoint()
        torch.cuda.synchronize()
        if ck == b.FP8_E4M3:
            got = back.view(torch.uint8).cpu().numpy().ravel()
            want = ro.e4m3_encode(vals.astype(np.float64).ravel())
            np.testing.assert_array_equal(got, want)
        else:
            got = back.view(torch.int16).cpu().numpy().ravel()
            want16 = vals.astype(np.float64).astype(np.float16).ravel()
            nan = np.isnan(want16)
            np.testing.assert_array_equal(got[~nan], want16.view(np.int16)[~nan])
            assert np.all(np.isnan(back.cpu().numpy().ravel()[nan]))
    # per-slot loads round the same way
    st = b.ReplayState(b.make_config(b.GDN, 3, H, H, C, R, 4, b.F32, ckpt_dtype=b.FP8_E4M3))
    st.load_slots([2, 0], torch.from_numpy(vals).cuda())
    back = st.read_checkpoint().view(torch.uint8).cpu().numpy()
    want = ro.e4m3_encode(vals.astype(np.float64)).reshape(vals.shape)
    np.testing.assert_array_equal(back[2], want[0])
    np.testing.assert_array_equal(back[0], want[1])
    assert not back[1].any()                         # the slot nobody loaded keeps its zero init


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_full_size_ragged_occupancy(kind):
    """The batch-256 layers with a seeded occupancy pattern: each step about 1/8 of the
    sequences sit out, every 8 steps 4 sequences leave and 4 new ones arrive by a per-slot
    load (prefill handoff); 40 steps.  Three sampled sequences (one of them re-loaded
    mid-window) are replayed by the oracle from copies of the device-drawn inputs."""
    from hybrid_decode_replay_amd import binding as b
    from oracle import replay_oracle as ro
    B, T, cap = 256, 40, 16
    if kind == "mamba2":
        H, G, C, R = 128, 8, 64, 128
        A, D = synth.mamba2_params(1, H)
        params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
        toks = synth.mamba2_tokens_device(11, T, B, H, G, C, R, "cuda")
        cfg = b.make_config(b.MAMBA2, B, H, G, C, R, cap, b.BF16)
    else:
        H, G, C, R = 32, 32, 128, 128
        params = None
        toks = synth.gdn_tokens_device(12, T, B, H, G, R, C, "cuda")
        cfg = b.make_config(b.GDN, B, H, G, C, R, cap, b.BF16)
    st = b.ReplayState(cfg)
    S0 = synth.checkpoint_device(13, (B, H, C, R), "cuda")
    st.load_checkpoint(S0)
    rng = np.random.default_rng(14)
    masks = rng.random((T, B)) >= 0.125
    sample = [3, 100, 254]
    arrivals = {}
    for t in range(8, T, 8):
        slots = sorted(set(rng.choice(B, size=4, replace=False).tolist()) | ({100} if t == 16 else set()))
        arrivals[t] = (slots, synth.checkpoint_device(15 + t, (len(slots), H, C, R), "cuda"))
    ys = torch.zeros((T, B, H, C), dtype=torch.bfloat16, device="cuda")
    print(f"[full-size ragged {kind}] launching", flush=True)
    for t in range(T):
        if t in arrivals:
            st.load_slots(*arrivals[t])
        st.decode({k: v[t:t + 1] for k, v in toks.items()}, params, y=ys[t:t + 1],
                  active=torch.from_numpy(masks[t].astype(np.uint8)).cuda())
    ck = st.read_checkpoint()
    L, Pd, F, E = st.read_book()
    torch.cuda.synchronize()
    S0s = S0[sample].cpu().numpy()
    sess = ro.Mamba2Session(A, D, S0s) if kind == "mamba2" else ro.GDNSession(S0s)
    host = {k: v[:, sample].float().cpu().numpy() for k, v in toks.items()}
    yg = ys[:, sample].float().cpu().numpy()
    for t in range(T):
        if t in arrivals:
            slots, Snew = arrivals[t]
            mine = [(i, sample.index(s)) for i, s in enumerate(slots) if s in sample]
            if mine:
                sess.load_slots([j for _, j in mine], Snew[[i for i, _ in mine]].cpu().numpy())
        m = masks[t][sample]
        yo = sess.decode(synth.token(host, t), active=m)
        if m.any():
            err = ro.normwise_error(yg[t][m], yo[m])
            assert err <= 2e-2, (t, err)
        assert not np.any(yg[t][~m]), t
    assert list(L.cpu().numpy()[sample]) == list(sess.len) and list(F.cpu().numpy()[sample]) == list(sess.fc)
    assert int(E[0]) == 0 and torch.all(Pd == 0)
    err_ck = ro.normwise_error(ck[sample].cpu().numpy(), sess.ckpt, axis=(2, 3))
    assert err_ck <= 1e-4, err_ck
