"""GPU runtime behaviour through the C ABI: HIP-graph capture and replay,
concurrent packing from several host threads, and launches on several
streams."""
import threading

import numpy as np
import pytest
import torch

import oracle
from sparse_matrix_vector_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_matrix_vector_amd as nm
    nm.lib()
    return nm


def bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def test_graph_capture_replays(nm):
    """nm_spmv, nm_spmv_multi and nm_gemv_dense captured into one graph; every
    replay (with unrelated eager work and synchronisations in between, and x
    changed between replays) must equal the eager result."""
    tdt = torch.float16
    K = 4096
    W1 = I.weight(512, K, tdt, 61, device="cuda")
    W2 = I.weight(256, K, tdt, 62, device="cuda")
    W3 = I.weight(1024, 14336, tdt, 63, device="cuda")
    p1, p2, p3 = nm.pack(W1, None, 2, 4), nm.pack(W2, None, 2, 4), nm.pack(W3, None, 2, 4)
    x = I.activation_normal(1, K, tdt, 64, device="cuda")
    xd = I.activation_normal(1, 14336, tdt, 65, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        ys = nm.spmv_multi([p1, p2], x, 2, 4)
        yd = nm.spmv(*p3, xd, 2, 4)
        yg = nm.gemv_dense(W1, x)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            ys = nm.spmv_multi([p1, p2], x, 2, 4)
            yd = nm.spmv(*p3, xd, 2, 4)
            yg = nm.gemv_dense(W1, x)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(5):
        x.copy_(I.activation_normal(1, K, tdt, 100 + rep, device="cuda"))
        junk = torch.randn(1 << 20, device="cuda").sum()       # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e1, e2 = nm.spmv_multi([p1, p2], x, 2, 4)
        assert torch.equal(ys[0].view(torch.int16), e1.view(torch.int16)), rep
        assert torch.equal(ys[1].view(torch.int16), e2.view(torch.int16)), rep
        assert torch.equal(yd.view(torch.int16), nm.spmv(*p3, xd, 2, 4).view(torch.int16)), rep
        assert torch.equal(yg.view(torch.int16), nm.gemv_dense(W1, x).view(torch.int16)), rep
        del junk


def test_concurrent_pack_from_threads(nm):
    """nm_pack is synchronous and serialises its device status word; packs
    issued from several host threads (each on its own stream) must all be
    byte-identical to the oracle."""
    tdt = torch.bfloat16
    jobs = [(I.weight(300 + 17 * i, 2048, tdt, 70 + i), (2, 4) if i % 2 else (4, 8)) for i in range(6)]
    results = [None] * len(jobs)
    errors = []

    def work(i):
        try:
            W, (n, m) = jobs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                v, mk = nm.pack(W.cuda(), None, n, m, stream=s)
            s.synchronize()
            results[i] = (bits(v), mk.cpu().numpy())
        except Exception as e:                      # noqa: BLE001 -- reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (W, (n, m)), (v, mk) in zip(jobs, results):
        ov, om = oracle.pack(bits(W), None, n, m, "bf16")
        assert np.array_equal(v, ov) and np.array_equal(mk, om)


def test_launches_on_several_streams(nm):
    tdt = torch.float16
    Ws = [I.weight(700, 4096, tdt, 80 + i, device="cuda") for i in range(4)]
    packs = [nm.pack(W, None, 2, 4) for W in Ws]
    x = I.activation_normal(2, 4096, tdt, 90, device="cuda")
    ref = [nm.spmv(v, m, x, 2, 4) for v, m in packs]
    streams = [torch.cuda.Stream() for _ in packs]
    outs = []
    for s, (v, m) in zip(streams, packs):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            outs.append(nm.spmv(v, m, x, 2, 4))
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
