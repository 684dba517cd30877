"""Host-side helpers of bench.py (no GPU): the code hash that decides whether a committed counter
summary still describes the current kernels."""

import bench


def test_code_only_drops_comments_and_layout_but_keeps_literals():
    src = ('int a;  // tail "quoted"\n/* block\n   comment */ const char* s = "//kept /* kept */";\n'
           "char q = '\"'; char e = '\\''; x  =\t1;")
    assert bench.code_only(src) == ('int a; const char* s = "//kept /* kept */"; '
                                    "char q = '\"'; char e = '\\''; x = 1;")


def test_kernel_hash_ignores_comments_and_follows_code(tmp_path, monkeypatch):
    f = tmp_path / "k.hip"
    monkeypatch.setitem(bench.KERNEL_SRCS, "k_probe", [str(f)])
    f.write_text("__global__ void k(float* p) { p[0] = 1.0f; }\n")
    h0 = bench.kernel_hash("k_probe")
    f.write_text("// what k does\n__global__ void k(float* p) {\n  p[0] = 1.0f;  /* one */\n}\n")
    assert bench.kernel_hash("k_probe") == h0
    f.write_text("__global__ void k(float* p) { p[0] = 2.0f; }\n")
    assert bench.kernel_hash("k_probe") != h0


def test_every_kernel_has_a_hash_over_existing_sources():
    import os
    for k, files in bench.KERNEL_SRCS.items():
        assert files and all(os.path.exists(f) for f in files), k
        assert len(bench.kernel_hash(k)) == 16


def test_mean_elements_per_launch_cover_the_shard():
    """Per-launch accounting is the mean over one step's launches, so launches x mean = the shard:
    GPT-3's 40 windows of 64 Mi and a 43,836,992-element tail, the offloaded 7B step's 25 chunks of
    32 Mi and a 3,441,152-element last chunk, and one launch for the whole-shard workloads."""
    cases = {"gpt3": (41, 2_728_191_552), "offload7b": (26, 842_301_952), "llama7b": (1, 842_301_952),
             "gpt2": (1, 15_544_608), "llama13b": (1, 813_491_520)}
    for w, (launches, S) in cases.items():
        assert round(bench.launch_elems(w) * launches) == S, w
    assert bench.algorithmic_bytes_per_launch("llama7b") == 842_301_952 * 42
    assert round(bench.algorithmic_bytes_per_launch("gpt3") * 41) == 2_728_191_552 * 154


def test_profiled_runs_skip_the_context_legs():
    """Every profiling command runs the bench with --no-context, so a trace holds only the timed
    step's launches (and, for the offloaded step, whole chunk sequences of the reduce kernel)."""
    for w in ("llama7b", "gpt2", "gpt3", "llama13b", "llama13b-clean", "gather7b", "offload7b"):
        cmds = bench.profile_commands(w)
        assert set(cmds) == {"trace", "fetch", "write", "plain"}
        for c in cmds.values():
            assert f"bench.py --workload {w} --no-context" in c, c


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "--gpus 2 is not supported" in capsys.readouterr().err
