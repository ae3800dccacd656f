"""Decode steps captured in a HIP graph and replayed (the serving loop's form:
the library launches on torch's current stream, which is the capture stream
inside torch.cuda.graph, so a captured step is the same kernel with the same
arguments).  Every replay is checked against the same steps run eagerly, with
eager work and synchronizations between replays."""
import numpy as np
import pytest

from weight_recurrent_memory_amd.inputs import decode_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_recurrent_memory_amd as fw  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fw.load_library()


@pytest.mark.parametrize("variant", [fw.FALCON_1, fw.FALCON_1A])
def test_decode_steps_replayed_from_a_graph(variant):
    N, H, dk, dv, pool, rounds = 16, 4, 64, 64, 4, 3
    d = decode_inputs(N, H, dk, dv, seed=1500 + variant, steps=pool)
    dev = "cuda"
    bf = torch.bfloat16
    up = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt).contiguous()
    qs, ks, vs = (up(d[n], bf) for n in ("q", "k", "v"))
    kw = dict(variant=variant, beta=0.5, lam=0.01, eps=1e-6)

    # eager: rounds x pool steps
    S_e, kp_e = up(d["S"], torch.float32), up(d["k_prev"], bf)
    outs_e = []
    for _ in range(rounds):
        for p in range(pool):
            outs_e.append(fw.decode_step(S_e, kp_e, qs[p], ks[p], vs[p], **kw).clone())
    states_e = (S_e.clone(), kp_e.clone())

    # graph: pool steps captured once, replayed `rounds` times
    S_g, kp_g = up(d["S"], torch.float32), up(d["k_prev"], bf)
    outs_g = torch.empty((pool, N, H, dv), device=dev, dtype=torch.float32)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for p in range(pool):
            fw.decode_step(S_g, kp_g, qs[p], ks[p], vs[p], out=outs_g[p], **kw)
    scratch = torch.zeros(1 << 20, device=dev)
    for r in range(rounds):
        g.replay()
        torch.cuda.synchronize()
        for p in range(pool):
            assert torch.equal(outs_g[p], outs_e[r * pool + p]), (r, p)
        scratch.add_(1.0)                  # eager work between replays
        torch.cuda.synchronize()
    assert torch.equal(S_g, states_e[0]) and torch.equal(kp_g, states_e[1])
