"""The floor probe (wsvd_floor_probe) is what the benchmark's `floors` object
times, so it must really read every byte it is given: in stream mode each
block's stored value is the xor of all 32-bit words of its share of the
buffer (masked to a finite float), checked bit for bit against the host; in
empty mode nothing is written unless the sentinel is present."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def W():
    from rank_kv_cache_flash_amd import wsvd
    wsvd.lib()
    return wsvd


@pytest.mark.parametrize("blocks,chunks", [(160, 1000), (3, 4096), (7, 1), (513, 257)])
def test_stream_probe_reads_every_word(W, blocks, chunks):
    rng = np.random.default_rng(blocks * 7919 + chunks)
    host = rng.integers(0, 2 ** 32, size=blocks * chunks * 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.uint8).copy()).cuda()
    sink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    print(f"[case] stream probe blocks={blocks} chunks={chunks}", flush=True)
    W.floor_probe(1, blocks, sink, src)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.reshape(blocks, chunks * 4), axis=1) & np.uint32(0x3F7FFFFF)
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want)


def test_empty_probe_writes_only_the_sentinel(W):
    blocks = 300
    vals = torch.arange(blocks, dtype=torch.float32, device="cuda") + 0.5
    vals[17] = 12345.0
    before = vals.clone()
    print(f"[case] empty probe blocks={blocks}", flush=True)
    W.floor_probe(0, blocks, vals)
    torch.cuda.synchronize()
    before[17] = 0.0
    assert torch.equal(vals, before)
