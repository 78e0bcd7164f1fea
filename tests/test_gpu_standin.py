"""GPU parity of the stand-in non-SSM layers (replay_standin_linear, replay_standin_attention)
against the fp64 references of oracle/standin_oracle.py.

These layers are the rest of a hybrid model's decode step ([TR] "NVIDIA ve Dao AI Lab
...", section "ReplaySSM nasil calisir?": SSM layers interleaved with attention
layers).  Inputs are seeded bf16 values; the reference sees exactly them.  Both
kernels accumulate in fp32 and round their outputs to bf16 (RNE), so an output row
is held to 1e-2 normwise (bf16 rounding 2^-9 plus fp32 accumulation error).
Shapes cover several tiles with ragged rows (M not a multiple of 256), cache lengths
below, at and past one 64-token chunk and past the four waves' stride, every grouped
query ratio, strided query rows, and the batch-256 shapes the benchmark times
(sampled rows).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_decode_replay_amd import binding  # noqa: F401  (fails loudly if not built)
    yield


def _bf16(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (std * torch.randn(shape, generator=g)).to(torch.bfloat16)


def _err(got, ref):
    from oracle import replay_oracle as ro
    return ro.normwise_error(got, ref)


@pytest.mark.parametrize("M,K,N", [(1, 128, 32), (37, 384, 96), (256, 1024, 256), (300, 512, 64), (256, 4096, 160),
                                   (129, 64, 40), (5, 192, 1), (256, 8192, 200), (200, 192, 16384)])
def test_linear(M, K, N):
    from hybrid_decode_replay_amd import binding as b
    from oracle import standin_oracle as so
    X, W = _bf16((M, K), M * 7 + K), _bf16((N, K), N + K, std=K ** -0.5)
    Y = b.standin_linear(X.cuda(), W.cuda())
    torch.cuda.synchronize()
    ref = so.linear(X.float().numpy(), W.float().numpy())
    err = _err(Y.float().cpu().numpy(), ref)
    print(f"[linear] M={M} K={K} N={N}: err {err:.2e}", flush=True)
    assert err <= TOL, err


def test_linear_rejects_bad_shapes():
    from hybrid_decode_replay_amd import binding as b
    X, W = _bf16((4, 100), 1).cuda(), _bf16((32, 100), 2).cuda()
    with pytest.raises(b.ReplayError) as e:
        b.standin_linear(X, W)
    assert e.value.status == b.ERR_SHAPE
    X, W = _bf16((4, 96), 1).cuda(), _bf16((40, 96), 2).cuda()
    with pytest.raises(b.ReplayError) as e:
        b.standin_linear(X, W)
    assert e.value.status == b.ERR_SHAPE


@pytest.mark.parametrize("B,Hq,Hkv,L", [(3, 8, 2, 1), (3, 8, 2, 63), (2, 8, 2, 64), (2, 8, 2, 65), (2, 4, 4, 300),
                                        (2, 8, 4, 257), (1, 8, 1, 1024), (4, 32, 8, 700)])
def test_attention(B, Hq, Hkv, L):
    from hybrid_decode_replay_amd import binding as b
    from oracle import standin_oracle as so
    D = 128
    extra = 24 if Hq == 8 else 0                       # a strided query row (as in a fused qkv output)
    qrow = _bf16((B, Hq * D + extra), B + Hq + L)
    Kc, Vc = _bf16((B, Hkv, L, D), L + 1), _bf16((B, Hkv, L, D), L + 2)
    scale = D ** -0.5
    o = b.standin_attention(qrow.cuda(), Kc.cuda(), Vc.cuda(), scale)
    torch.cuda.synchronize()
    q = qrow[:, :Hq * D].reshape(B, Hq, D).float().numpy()
    ref = so.attention(q, Kc.float().numpy(), Vc.float().numpy(), scale)
    err = _err(o.float().cpu().numpy(), ref)
    print(f"[attention] B={B} Hq={Hq} Hkv={Hkv} L={L}: err {err:.2e}", flush=True)
    assert err <= TOL, err


def test_attention_rejects_unsupported():
    from hybrid_decode_replay_amd import binding as b
    q = _bf16((2, 3 * 128), 1).cuda()
    Kc = _bf16((2, 1, 4, 128), 2).cuda()
    with pytest.raises(b.ReplayError) as e:
        b.standin_attention(q, Kc, Kc, 1.0)            # 3 query heads per key/value head
    assert e.value.status == b.ERR_UNSUPPORTED
    Kc64 = _bf16((2, 1, 4, 64), 3).cuda()
    with pytest.raises(b.ReplayError) as e:
        b.standin_attention(_bf16((2, 64), 4).cuda(), Kc64, Kc64, 1.0)
    assert e.value.status == b.ERR_UNSUPPORTED


def test_full_size_standins_sampled():
    """The benchmark's shapes: a batch-256 projection 4096 -> 18560 and attention over 2048
    cached tokens with 32 query and 8 key/value heads; sampled rows and sequences."""
    from hybrid_decode_replay_amd import binding as b
    from oracle import standin_oracle as so
    M, K, N = 256, 4096, 18560
    g = torch.Generator(device="cuda").manual_seed(5)
    X = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    W = (torch.randn((N, K), generator=g, device="cuda") * K ** -0.5).to(torch.bfloat16)
    Y = b.standin_linear(X, W)
    torch.cuda.synchronize()
    rows = [0, 77, 255]
    cols = np.arange(0, N, 37)
    ref = so.linear(X[rows].float().cpu().numpy(), W[cols].float().cpu().numpy())
    err = _err(Y[rows][:, cols].float().cpu().numpy(), ref)
    assert err <= TOL, err
    B, Hq, Hkv, L, D = 256, 32, 8, 2048, 128
    q = torch.randn((B, Hq * D), generator=g, device="cuda").to(torch.bfloat16)
    Kc = torch.randn((B, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
    Vc = torch.randn((B, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
    o = b.standin_attention(q, Kc, Vc, D ** -0.5)
    torch.cuda.synchronize()
    seqs = [0, 100, 255]
    ref = so.attention(q[seqs].reshape(3, Hq, D).float().cpu().numpy(), Kc[seqs].float().cpu().numpy(),
                       Vc[seqs].float().cpu().numpy(), D ** -0.5)
    err = _err(o[seqs].float().cpu().numpy(), ref)
    assert err <= TOL, err
