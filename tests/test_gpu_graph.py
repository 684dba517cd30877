"""The library's launches captured into a HIP graph (torch.cuda.graph) and replayed: every replay,
with eager work and synchronisations between replays, must give the same bits as the same calls
made eagerly. The step's fp32 constants are fixed at capture (one value of t)."""

import pytest
import torch

import zero_partition_plan_amd as Z
from gpu_util import DEV, assert_bits_equal, bits16, bits32

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=5)


def _state(seed, n, R):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    reps = (torch.randn(R, n, generator=g, device=DEV) * 1e-3).to(torch.bfloat16)
    master = torch.randn(n, generator=g, device=DEV) * 0.02
    m = torch.randn(n, generator=g, device=DEV) * 1e-4
    v = torch.rand(n, generator=g, device=DEV) * 1e-7
    return reps, master, m, v


@pytest.mark.parametrize("n", [256 * 1000, 256 * 1000 + 77])
def test_fused_step_graph_replays_match_eager(n):
    R = 8
    reps, master, m, v = _state(1, n, R)
    eager = [t.clone() for t in (master, m, v)]
    e_out = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    g_state = [t.clone() for t in (master, m, v)]
    g_out = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    h = Z.adam_hparams(**HP)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm the library (device attributes) off-capture
        Z.zero_adam_shard_step(reps, 0, 1.0, g_state[0], g_state[1], g_state[2], h)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        Z.zero_adam_shard_step(reps, n, 1.0, g_state[0], g_state[1], g_state[2], h, out=g_out)
    scratch = torch.randn(1 << 20, device=DEV)
    for k in range(3):
        graph.replay()
        scratch.mul_(1.0001).add_(0.5)            # unrelated eager work between replays
        torch.cuda.synchronize()
        Z.zero_adam_shard_step(reps, n, 1.0, eager[0], eager[1], eager[2], h, out=e_out)
        torch.cuda.synchronize()
        for a, b, what in zip(g_state, eager, ("master", "m", "v")):
            assert_bits_equal(bits32(a), bits32(b), f"replay {k} {what}")
        assert_bits_equal(bits16(g_out), bits16(e_out), f"replay {k} params")


@pytest.mark.parametrize("device_clip", [False, True])
def test_reduce_sqnorm_skip_graph_replays_match_eager(device_clip):
    """Pass 1, the squared-norm finish and pass 2 with the device skip flag, in one graph. The flag
    is cleared by a fill kernel inside the graph (not a memset). With ``device_clip`` the clip
    scale is formed on the device between the passes (zero_clip_scale), so the graph holds the
    whole clipped step and each replay clips by that replay's own norm."""
    n, R = 512 * 300 + 5, 16
    g = torch.Generator(device=DEV)
    g.manual_seed(2)
    reps = (torch.randn(R, n, generator=g, device=DEV) * 1e-4 * 65536).to(torch.float16)
    master = torch.randn(n, generator=g, device=DEV) * 0.02
    zeros = torch.zeros(n, device=DEV)

    def buffers():
        return dict(p=master.clone(), m=zeros.clone(), v=zeros.clone(), g=torch.empty(n, device=DEV),
                    flag=torch.zeros(1, dtype=torch.int32, device=DEV),
                    parts=torch.empty(Z.zero_sq_partials_len(n), dtype=torch.float64, device=DEV),
                    sq=torch.empty(1, dtype=torch.float64, device=DEV),
                    gs=torch.empty(1, dtype=torch.float32, device=DEV),
                    out=torch.zeros(n, dtype=torch.float16, device=DEV))

    h = Z.adam_hparams(step=1, lr=1e-3, weight_decay=0.01)

    def step(b):
        b["flag"].fill_(0)
        Z.zero_reduce_shard(reps, n, b["g"], b["flag"], b["parts"], 2.0 ** -16)
        Z.zero_shard_sqnorm(None, n, 2.0 ** -16, b["parts"], b["sq"])
        if device_clip:
            Z.zero_clip_scale(b["sq"], 0.01, 1e-6, 2.0 ** -16, b["gs"])
            Z.zero_adam_shard_step_dev_scale([b["g"]], n, b["gs"], b["p"], b["m"], b["v"], h,
                                             out=b["out"], skip=b["flag"])
        else:
            Z.zero_adam_shard_step([b["g"]], n, 2.0 ** -16, b["p"], b["m"], b["v"], h, out=b["out"],
                                   skip=b["flag"])

    gb, eb = buffers(), buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(buffers())
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gb)
    for k in range(3):
        graph.replay()
        torch.cuda.synchronize()
        step(eb)
        torch.cuda.synchronize()
        for key in ("p", "m", "v", "g", "out"):
            a, b = gb[key], eb[key]
            assert torch.equal(a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                               b.view(torch.int16 if b.element_size() == 2 else torch.int32)), (k, key)
        assert float(gb["sq"].item()) == float(eb["sq"].item()) and int(gb["flag"].item()) == 0
        if device_clip:
            assert gb["gs"].view(torch.int32).item() == eb["gs"].view(torch.int32).item()
            coef = min(1.0, 0.01 / (float(gb["sq"].item()) ** 0.5 + 1e-6))
            assert 0.0 < coef < 1.0                     # clipping is active


@pytest.mark.parametrize("static", [False, True])
def test_clipped_step_with_device_counter_replays_as_successive_steps(static):
    """The whole clipped two-pass step (flag fill, reduce, squared norm, clip scale, update with t
    from a device counter, t advance) captured once: each replay is the next training step. Replays
    match eager steps with t from the host, bit for bit; an overflow written into a replica between
    replays makes that replay skip, with t not advancing. With ``static`` the captured step's
    reduce and norm are zero_reduce_shard_static (no workspace; the partials in the library's own
    scratch), which is what a caller that cannot allocate captures; the eager steps keep the
    workspace pair."""
    n, R, ls = 256 * 700 + 9, 16, 2.0 ** 16
    g = torch.Generator(device=DEV)
    g.manual_seed(4)
    reps = (torch.randn(R, n, generator=g, device=DEV) * 1e-4 * ls).to(torch.float16)
    master = torch.randn(n, generator=g, device=DEV) * 0.02
    kw = dict(lr=1e-3, weight_decay=0.01)
    table = Z.adam_table(Z.adam_hparams(**kw), 64, device=DEV)

    def buffers():
        return dict(p=master.clone(), m=torch.zeros(n, device=DEV), v=torch.zeros(n, device=DEV),
                    g=torch.empty(n, device=DEV), flag=torch.zeros(1, dtype=torch.int32, device=DEV),
                    parts=torch.empty(Z.zero_sq_partials_len(n), dtype=torch.float64, device=DEV),
                    sq=torch.empty(1, dtype=torch.float64, device=DEV),
                    gs=torch.empty(1, dtype=torch.float32, device=DEV),
                    t=torch.ones(1, dtype=torch.int64, device=DEV),
                    status=torch.zeros(1, dtype=torch.int32, device=DEV),
                    out=torch.zeros(n, dtype=torch.float16, device=DEV))

    def front(b, use_static=False):
        b["flag"].fill_(0)
        if use_static:
            Z.zero_reduce_shard_static(reps, n, b["g"], b["flag"], b["sq"], 1.0 / ls)
        else:
            Z.zero_reduce_shard(reps, n, b["g"], b["flag"], b["parts"], 1.0 / ls)
            Z.zero_shard_sqnorm(None, n, 1.0 / ls, b["parts"], b["sq"])
        Z.zero_clip_scale(b["sq"], 0.01, 1e-6, 1.0 / ls, b["gs"])

    def graph_step(b):
        front(b, static)
        Z.zero_adam_shard_step_dev_t([b["g"]], n, b["gs"], table, b["t"], b["status"], b["p"], b["m"],
                                     b["v"], out=b["out"], skip=b["flag"])

    gb, eb = buffers(), buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph_step(buffers())
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graph_step(gb)
    t_host = 1
    saved = reps[3, 77].clone()
    for k in range(5):
        inject = k == 2
        if inject:
            reps[3, 77] = float("inf")
        graph.replay()
        torch.cuda.synchronize()
        front(eb)                                      # the eager step, t from the host
        Z.zero_adam_shard_step_dev_scale([eb["g"]], n, eb["gs"], eb["p"], eb["m"], eb["v"],
                                         Z.adam_hparams(step=t_host, **kw), out=eb["out"], skip=eb["flag"])
        torch.cuda.synchronize()
        if inject:
            reps[3, 77] = saved
            assert int(gb["flag"].item()) == 1
        else:
            t_host += 1
        assert int(gb["t"].item()) == t_host, k
        for key in ("p", "m", "v", "g", "out"):
            a, b = gb[key], eb[key]
            assert torch.equal(a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                               b.view(torch.int16 if b.element_size() == 2 else torch.int32)), (k, key)
        assert gb["gs"].view(torch.int32).item() == eb["gs"].view(torch.int32).item(), k
    assert t_host == 5 and int(gb["status"].item()) == 0
