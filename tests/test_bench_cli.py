"""CPU checks of the benchmark's command line and of the source hashes that
decide whether a stored traffic measurement still describes a kernel."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _bench(env_extra={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present")
def test_without_a_gpu_it_fails_loudly():
    r = _bench("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode != 0
    assert r.stdout == ""


def test_bench_and_profiling_hash_the_same_sources():
    sys.path.insert(0, ROOT)
    import bench
    from exact_tiled_attention_04_amd import profiling
    assert bench.FWD_SOURCES == profiling.FWD_SOURCES
    assert bench.FP8_SOURCES == profiling.FP8_SOURCES
    assert bench.kernel_source_hash(bench.FWD_SOURCES) == profiling.kernel_source_hash(profiling.FWD_SOURCES)
    assert bench.kernel_source_hash(bench.FP8_SOURCES) == profiling.kernel_source_hash(profiling.FP8_SOURCES)
    # every kernel family hashes its own files
    assert profiling.sources_of("bwd_dkdv_kernel") == profiling.BWD_SOURCES
    assert profiling.sources_of("decode_split") == profiling.DECODE_SOURCES
    assert profiling.sources_of("fwd_fp8") == profiling.FP8_SOURCES
    assert profiling.sources_of("fwd_f32_kernel") == profiling.F32_SOURCES == bench.F32_SOURCES
    assert profiling.sources_of("fwd_") == profiling.FWD_SOURCES
    for srcs in (profiling.FWD_SOURCES, profiling.FP8_SOURCES, profiling.BWD_SOURCES, profiling.DECODE_SOURCES):
        for fn in srcs:
            assert os.path.exists(os.path.join(ROOT, "exact_tiled_attention_04_amd", "csrc", fn)), fn


def test_stored_traffic_files_are_well_formed():
    prof = os.path.join(ROOT, "profiles")
    for fn in sorted(os.listdir(prof)):
        if fn.startswith("traffic_") and fn.endswith(".json"):
            rec = json.load(open(os.path.join(prof, fn)))
            assert rec["workload"] == fn[len("traffic_"):-len(".json")]
            assert len(rec["kernel_source_sha256"]) == 64
            assert rec["hbm_bytes_per_launch"] == pytest.approx(rec["fetch_bytes"] + rec["write_bytes"], abs=2)
            assert rec["commands"] and all("rocprofv3" in c for c in rec["commands"])


def test_calibration_uses_only_the_large_copy(tmp_path, monkeypatch):
    """A small copy in the same counter run must not dilute the calibration
    factor: only the copies with the largest grid count."""
    from exact_tiled_attention_04_amd import profiling
    rows = [("1", "__amd_rocclr_copyBuffer", "512", "3.0"),
            ("2", "__amd_rocclr_copyBuffer", "131072", "524300.0"),
            ("3", "void fa::(anonymous namespace)::decode_split_kernel<>", "64", "1000.0"),
            ("4", "__amd_rocclr_copyBuffer", "131072", "524298.0")]
    with open(tmp_path / "run_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n")
        for disp, name, grid, val in rows:
            f.write(f'{disp},"{name}",{grid},FETCH_SIZE,{val}\n')
    monkeypatch.setattr(profiling, "KERNEL_KEY", "decode_split")
    attn, copy = profiling.counter_per_dispatch(str(tmp_path))
    assert copy["FETCH_SIZE"] == [524300.0, 524298.0]
    assert attn["FETCH_SIZE"] == [1000.0]


def test_clock_adjusted_fraction():
    """The line prices the achieved rate against the peak scaled to the clock
    read during the timed calls (matrix- and ALU-bound kernels only)."""
    import bench
    t = {"sclk_mhz": {"mean": 1800.0, "samples": 3}, "warm_s": 1.0}
    out = bench.clock_fields(t, {"rate_at_avg": 1000.0}, 2400.0, "mfma")
    assert out["frac_of_peak_at_measured_clock"] == round(1000.0 / (2400.0 * 1800.0 / 2400.0), 4)
    assert "frac_of_peak_at_measured_clock" not in bench.clock_fields(t, {"rate_at_avg": 5.0}, 8000.0, "hbm")
    assert "frac_of_peak_at_measured_clock" not in bench.clock_fields(
        {"sclk_mhz": None, "warm_s": 1.0}, {"rate_at_avg": 1.0}, 1.0, "mfma")
    assert "frac_of_peak_at_measured_clock" not in bench.clock_fields(
        {"sclk_mhz": {"error": "no amdsmi"}, "warm_s": 1.0}, {"rate_at_avg": 1.0}, 1.0, "mfma")


def test_power_reading_passes_through():
    """Socket power read during the timed calls (with the board's cap) is
    carried into the line's clock object when the driver reports it."""
    import bench
    pw = {"mean": 1370.0, "samples": 4, "cap": 1400.0, "source": "amdsmi"}
    t = {"sclk_mhz": {"mean": 1800.0, "samples": 3}, "warm_s": 1.0, "power_w": pw}
    assert bench.clock_fields(t, {"rate_at_avg": 1.0}, 2400.0, "mfma")["power_w"] == pw
    t["power_w"] = None
    assert "power_w" not in bench.clock_fields(t, {"rate_at_avg": 1.0}, 2400.0, "mfma")
    assert "power_w" not in bench.clock_fields({"sclk_mhz": None, "warm_s": 1.0}, {"rate_at_avg": 1.0}, 1.0, "hbm")
