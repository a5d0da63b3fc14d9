"""moe_layer_decode_static (the entry point that allocates nothing: its per-call
scratch is the library's static device array) against moe_layer_decode on the
same inputs, through the C ABI: routing, bookkeeping and outputs must be the
same bits, on consecutive calls whose second is smaller than the first; the
oracle checks the same steps.  Also its argument limits."""
import numpy as np
import pytest

from oracle import OracleLayer
from synth import CONFIGS, WorkloadConfig, activations, global_scales

from gpu_util import OracleBlobs, check_output, log, make_cache, torch_cuda

pytestmark = pytest.mark.gpu


def _pair(cfg, max_rows, slots):
    a = make_cache(cfg, max_rows=max_rows, slots=slots)
    b = make_cache(cfg, max_rows=max_rows, slots=slots)
    return a, b


def _step(torch, B, sc, static, z, x_bits):
    M = z.shape[0]
    d_z = torch.from_numpy(np.ascontiguousarray(z, np.float32)).cuda()
    d_x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()
    d_y = torch.full((M, sc.hidden), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    fn = B.moe_layer_decode_static if static else B.moe_layer_decode
    fn(sc.h, 0, d_z.data_ptr(), d_x.data_ptr(), M, d_y.data_ptr(), s)
    ids, w, byp = sc.read_routing()
    return d_y.cpu().numpy(), ids, w, byp


SHAPES = {
    "tiny": (CONFIGS["tiny"], 16, 8, [8, 3, 16, 1, 5, 2]),
    "glm48": (WorkloadConfig("glm48", 6144, 2048, 48, 8, 32, 16, 6, routing="normal", seed=5), 16, 32,
              [16, 1, 4, 2, 8, 1]),
}


@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_static_entry_point_matches_the_workspace_one(shape):
    from hbm_expert_slot_amd import binding as B
    torch = torch_cuda()
    cfg, max_rows, slots, rows = SHAPES[shape]
    log("static scratch entry point: %s, M sequence %s" % (shape, rows))
    a, b = _pair(cfg, max_rows, slots)
    orc = OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, slots, OracleBlobs(cfg),
                      global_scales(cfg, 0, "unit"), keep_slot_bytes=False)
    rng = np.random.default_rng(17)
    for t, M in enumerate(rows):
        z = rng.standard_normal((M, cfg.n_experts)).astype(np.float32)
        z[:, :3] += 1.0                       # shared favourites: rows share experts
        x = activations(cfg, 0, t, M)
        ya, ia, wa, ba = _step(torch, B, a, False, z, x)
        yb, ib, wb, bb = _step(torch, B, b, True, z, x)
        assert np.array_equal(ia, ib) and np.array_equal(wa, wb) and ba == bb, (t, M)
        assert np.array_equal(ya, yb), (t, M)                 # same kernels, same bits
        for u, v in zip(a.read_state(0), b.read_state(0)):
            assert np.array_equal(u, v), (t, M)
        y_o, rec, ids_o, _ = orc.decode(z, x, with_output=(t < 3 or shape == "tiny"))
        assert np.array_equal(ib, ids_o), (t, M)
        if y_o is not None:
            check_output(yb, y_o, (t, M))
    sa, sb = a.stats(0), b.stats(0)
    assert sa == sb and sb["misses"] > 0 and sb["device_error"] == 0
    a.close()
    b.close()


def test_static_entry_point_limits():
    from hbm_expert_slot_amd import binding as B
    torch = torch_cuda()
    log("static scratch entry point: limits")
    cfg = CONFIGS["tiny"]
    sc = make_cache(cfg, max_rows=32)
    z = torch.zeros((32, cfg.n_experts), dtype=torch.float32, device="cuda")
    x = torch.zeros((32, cfg.hidden), dtype=torch.int16, device="cuda")
    y = torch.zeros((32, cfg.hidden), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for M in (0, 17, 32, 33):                 # prefill chunks need the caller's workspace
        with pytest.raises(B.SlotCacheError) as ei:
            B.moe_layer_decode_static(sc.h, 0, z.data_ptr(), x.data_ptr(), M, y.data_ptr(), s)
        assert ei.value.status == B.SC_E_ARG
    assert sc.stats(0)["steps"] == 0
    B.moe_layer_decode_static(sc.h, 0, z.data_ptr(), x.data_ptr(), 16, y.data_ptr(), s)
    assert sc.stats(0)["steps"] == 1
    sc.close()
    # a configuration whose per-call scratch exceeds the static array: 16 rows x 32 picks x H 8192 fp32
    # per-pick outputs alone are 16 MiB
    big = WorkloadConfig("big", 8192, 256, 32, 32, 32, 16, 1, routing="normal", seed=3)
    sc = make_cache(big, max_rows=16)
    z = torch.zeros((1, big.n_experts), dtype=torch.float32, device="cuda")
    x = torch.zeros((1, big.hidden), dtype=torch.int16, device="cuda")
    y = torch.zeros((1, big.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(B.SlotCacheError) as ei:
        B.moe_layer_decode_static(sc.h, 0, z.data_ptr(), x.data_ptr(), 1, y.data_ptr(), s)
    assert ei.value.status == B.SC_E_ARG and "static array" in str(ei.value)
    B.moe_layer_decode(sc.h, 0, z.data_ptr(), x.data_ptr(), 1, y.data_ptr(), s)   # the workspace path still runs
    assert sc.stats(0)["steps"] == 1
    sc.close()


def test_static_entry_point_under_graph_capture():
    """The use it is for: steps captured into a HIP graph through the static entry point,
    replayed three times, each replay checked against the same steps run eagerly through
    the workspace entry point on a second handle (outputs, routing state, counters)."""
    from hbm_expert_slot_amd import binding as B
    torch = torch_cuda()
    cfg = CONFIGS["tiny"]
    log("static scratch entry point under graph capture: tiny, 6 steps of 1-4 rows, 3 replays")
    a, b = _pair(cfg, 4, cfg.slots)
    rng = np.random.default_rng(29)
    rows = [1, 4, 2, 1, 3, 1]
    zs = [torch.from_numpy(rng.standard_normal((M, cfg.n_experts)).astype(np.float32)).cuda() for M in rows]
    xs = [torch.from_numpy(activations(cfg, 0, t, M).view(np.int16)).cuda() for t, M in enumerate(rows)]
    ya = [torch.zeros((M, cfg.hidden), dtype=torch.float32, device="cuda") for M in rows]
    yb = [torch.zeros((M, cfg.hidden), dtype=torch.float32, device="cuda") for M in rows]
    gstream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(gstream):
        g.capture_begin()
        for t, M in enumerate(rows):
            B.moe_layer_decode_static(a.h, 0, zs[t].data_ptr(), xs[t].data_ptr(), M, ya[t].data_ptr(),
                                      gstream.cuda_stream)
        g.capture_end()
    torch.cuda.synchronize()
    assert a.stats(0)["steps"] == 0            # capture enqueues nothing
    s = torch.cuda.current_stream().cuda_stream
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for t, M in enumerate(rows):
            B.moe_layer_decode(b.h, 0, zs[t].data_ptr(), xs[t].data_ptr(), M, yb[t].data_ptr(), s)
        torch.cuda.synchronize()
        for t in range(len(rows)):
            assert torch.equal(ya[t], yb[t]), (rep, t)
        for u, v in zip(a.read_state(0), b.read_state(0)):
            assert np.array_equal(u, v), rep
        assert a.stats(0) == b.stats(0), rep
    assert b.stats(0)["misses"] > 0
    a.close()
    b.close()
