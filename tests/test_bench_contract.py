"""Host checks of bench.py's command-line contract (no GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_summaries_pick_the_calibration_multiply(tmp_path):
    """The HBM-counter scaling uses the one float scalar multiply of the bench's
    calibration copy, not any other elementwise kernel of the run."""
    sys.path.insert(0, ROOT)
    import bench
    names = ["at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, x>",
             "at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, "
             "float, at::native::binary_internal::MulFunctor<float> >, std::array<char*, 2ul> >",
             "sffn::k_gate_up_t1<5, 1>(...)"]
    rows = {"FETCH_SIZE": [(names[0], 0.0), (names[1], 131072.0), (names[2], 19760.0)],
            "WRITE_SIZE": [(names[0], 4194304.0), (names[1], 262144.0), (names[2], 77.0)]}

    def fake_rows(d, q):
        return [(n, c, v, 1) for c, lst in rows.items() if c in d for n, v in lst]
    orig = bench._rocpd_rows
    bench._rocpd_rows = fake_rows
    try:
        out = str(tmp_path / "pmc.json")
        bench.summarize_pmc("FETCH_SIZE", "WRITE_SIZE", "k_gate_up_t1", out, "cmd")
        import json
        d = json.load(open(out))
        assert abs(d["fetch"]["scale"] - 2.0) < 1e-9 and abs(d["write"]["scale"] - 1.0) < 1e-9
    finally:
        bench._rocpd_rows = orig
