"""GPU parity of the ZeRO-3 parameter gather against the oracle (bit for bit: it is a copy)."""

import numpy as np
import pytest
import torch

import oracle as O
import zero_partition_plan_amd as Z
import fullshard as FS
from gpu_util import DEV, banner
from workloads import WORKLOADS, layer_ranges

pytestmark = pytest.mark.gpu


def _shards(rng, nd, S, eb, offset=0):
    """nd device shards (int16 or int32 bit patterns), each starting `offset` elements into its
    own allocation (to reach unaligned sources), and their host copies."""
    dt_np, dt_t = (np.int16, torch.int16) if eb == 2 else (np.int32, torch.int32)
    host = [rng.integers(-(1 << 15), 1 << 15, S).astype(dt_np) if eb == 2
            else rng.integers(-(1 << 31), 1 << 31, S, dtype=np.int64).astype(dt_np) for _ in range(nd)]
    dev = [torch.from_numpy(np.concatenate([np.zeros(offset, dt_np), h])).to(DEV)[offset:] for h in host]
    return host, dev


def _gather(dev_shards, begin, count, eb, out_offset=0, fill=-5):
    dt = torch.int16 if eb == 2 else torch.int32
    buf = torch.full((count + out_offset + 3,), fill, dtype=dt, device=DEV)
    Z.zero_gather_params(dev_shards, begin, count, buf[out_offset:out_offset + count])
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert (h[:out_offset] == fill).all() and (h[out_offset + count:] == fill).all(), "write outside out"
    return h[out_offset:out_offset + count]


def _ranges(S, nd):
    P = S * nd
    cands = {(0, P), (0, 0), (0, 1), (P - 1, 1), (3, min(P - 3, 2 * S)), (S - 1, 2), (S // 2, S),
             (1, P - 2), (S + 5, max(0, min(P - S - 5, 5000))), (max(0, P - 2 * S - 1), min(P, 2 * S + 1))}
    return sorted((b, c) for b, c in cands if 0 <= b and c >= 0 and b + c <= P)


@pytest.mark.parametrize("eb", [2, 4])
@pytest.mark.parametrize("nd,S", [(1, 1000), (3, 7), (8, 4096 + 3), (8, 100_000), (64, 2049), (5, 1)])
def test_gather_matches_oracle(nd, S, eb):
    banner(f"gather nd={nd} S={S} eb={eb}")
    rng = np.random.default_rng(nd * 31 + S + eb)
    host, dev = _shards(rng, nd, S, eb)
    for begin, count in _ranges(S, nd):
        got = _gather(dev, begin, count, eb)
        want = O.gather_range(host, begin, count)
        assert np.array_equal(got, want), (begin, count)


@pytest.mark.parametrize("src_off,out_off", [(1, 0), (0, 1), (3, 5), (8, 8)])
def test_gather_unaligned(src_off, out_off):
    rng = np.random.default_rng(src_off * 10 + out_off)
    nd, S = 4, 3 * 1024 + 17
    host, dev = _shards(rng, nd, S, 2, offset=src_off)
    for begin, count in ((0, nd * S), (S - 9, S + 20), (7, 5 * 1024)):
        got = _gather(dev, begin, count, 2, out_offset=out_off)
        assert np.array_equal(got, O.gather_range(host, begin, count)), (begin, count)


def test_gather_skips_untouched_null_shards_and_checks_errors():
    rng = np.random.default_rng(9)
    host, dev = _shards(rng, 4, 1000, 2)
    part = [None, dev[1], dev[2], None]
    assert np.array_equal(_gather(part, 1500, 900, 2), O.gather_range(host, 1500, 900))
    with pytest.raises(Z.ZeroError):                 # range needs shard 0
        _gather(part, 900, 200, 2)
    with pytest.raises(Z.ZeroError):                 # past the end
        _gather(dev, 3900, 101, 2)
    with pytest.raises(Z.ZeroError):                 # out inside a shard it reads
        Z.zero_gather_params(dev, 0, 100, dev[0][10:110])


def _oracle_window(shards, j0, j1, S):
    """The oracle's gather of flat [j0, j1) from downloaded shard pieces. A window touches at most
    two shards here; their pieces are placed at the end of one oracle shard and the start of the
    next (equal length), so the oracle's end-to-end layout reproduces the flat positions."""
    r0, r1 = j0 // S, (j1 - 1) // S
    assert r1 - r0 <= 1
    if r0 == r1:
        piece = shards[r0][j0 - r0 * S:j1 - r0 * S].cpu().numpy()
        return O.gather_range([piece], 0, j1 - j0)
    tail = shards[r0][j0 - r0 * S:].cpu().numpy()
    head = shards[r1][:j1 - r1 * S].cpu().numpy()
    L = max(len(tail), len(head))
    A = np.concatenate([np.zeros(L - len(tail), tail.dtype), tail])
    B = np.concatenate([head, np.zeros(L - len(head), head.dtype)])
    return O.gather_range([A, B], L - len(tail), j1 - j0)


@pytest.mark.timeout(900)
def test_llama7b_layers_from_eight_shards_full_size():
    """The Llama-7B flat bf16 parameters over 8 ranks (S = 842,301,952): every layer (embeddings,
    32 blocks, final norm and head) gathered in turn into a layer buffer, the next layer on a second
    stream while the current one is read (prefetch into the other of two buffers). Every element of
    every layer (all 6,738,415,616) is checked against the oracle's gather, in 16 Mi chunks on host
    threads; every shard boundary falls inside some layer."""
    w = WORKLOADS["llama7b"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    S = plan.shard_elems
    banner(f"llama7b gather S={S}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(21)
    flat = torch.randint(-(1 << 15), 1 << 15, (plan.padded_n,), generator=gen, dtype=torch.int16,
                         device=DEV)
    shards = [flat[r * S:(r + 1) * S] for r in range(w.nd)]
    layers = layer_ranges("llama-7b")
    biggest = max(e - s for _, s, e in layers)
    bufs = [torch.empty(biggest, dtype=torch.int16, device=DEV) for _ in range(2)]
    side, main = torch.cuda.Stream(), torch.cuda.current_stream()
    ready = [torch.cuda.Event(), torch.cuda.Event()]
    Z.zero_gather_params(shards, layers[0][1], layers[0][2] - layers[0][1], bufs[0], stream=side)
    ready[0].record(side)
    crossings = checked = 0
    for i, (name, a, b) in enumerate(layers):
        cur = bufs[i % 2]
        main.wait_event(ready[i % 2])
        if i + 1 < len(layers):
            _, a2, b2 = layers[i + 1]
            side.wait_stream(main)              # the other buffer's previous layer has been read
            Z.zero_gather_params(shards, a2, b2 - a2, bufs[(i + 1) % 2], stream=side)
            ready[(i + 1) % 2].record(side)
        n = b - a
        crossings += sum(1 for r in range(1, w.nd) if a < r * S < b)

        def work(lo, hi, cur=cur, a=a, name=name):
            got = cur[lo:hi].cpu().numpy()
            want = _oracle_window(shards, a + lo, a + hi, S)
            assert np.array_equal(got, want), (name, lo, hi)

        done, _ = FS.run_chunks(n, work)
        assert done == n, name
        checked += n
    torch.cuda.synchronize()
    assert crossings == w.nd - 1               # every internal boundary was crossed by some layer
    assert checked == w.n
    banner(f"llama7b gather: {checked} elements of {len(layers)} layers checked")
    del flat, shards, bufs
    torch.cuda.empty_cache()
