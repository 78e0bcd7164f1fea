"""GPU checks of the streaming kernels behind the in-run bandwidth ceilings: the copy
moves every byte (and none past the end), and the read's per-tile sums equal the sums
of the fp32 values of each 32 KiB tile, the last tile ragged."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("nbytes", [16, 4096, 32768, 32768 * 9 + 48, 1 << 22])
def test_stream_copy_moves_every_byte(nbytes):
    from hybrid_decode_replay_amd import binding as b
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randn(nbytes // 4 + 64, generator=g).cuda()
    dst = torch.full_like(src, float("nan"))
    b.stream_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    n = nbytes // 4
    assert torch.equal(dst[:n], src[:n])
    assert torch.isnan(dst[n:]).all(), "wrote past the end"


@pytest.mark.parametrize("nbytes", [16, 32768, 32768 * 5 + 48, 32768 * 64, (1 << 24) + 32768 * 3 + 16 * 7])
def test_stream_read_tile_sums(nbytes):
    from hybrid_decode_replay_amd import binding as b
    g = torch.Generator(device="cpu").manual_seed(7 + nbytes)
    host = torch.randn(nbytes // 4, generator=g)
    src = host.cuda()
    parts = torch.full((b.stream_read_partials(nbytes) + 4,), float("nan"), device="cuda")
    b.stream_read(src, nbytes, parts)
    torch.cuda.synchronize()
    got = parts.cpu().numpy().astype(np.float64)
    k = b.stream_read_partials(nbytes)
    x = host.numpy().astype(np.float64)
    per = b.STREAM_TILE_BYTES // 4
    want = np.array([x[i * per:(i + 1) * per].sum() for i in range(k)])
    scale = np.array([np.abs(x[i * per:(i + 1) * per]).sum() for i in range(k)])
    assert np.all(np.abs(got[:k] - want) <= 1e-5 * scale + 1e-6)
    assert np.isnan(got[k:]).all(), "wrote past the last tile's sum"
