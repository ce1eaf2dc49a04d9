"""Host-side pieces of bench.py: the JSON contract's fixed fields and the rule
that counter traffic is reported only for the kernel instance it was taken on."""
import json

import pytest

import bench


KERNELS = ("adam_kernel", "adam_db_kernel", "fold_adam_db_kernel")


def _kernel_of(rec):
    return rec["kernel"].split("<")[0].split()[-1]


def test_traffic_only_for_the_profiled_instance():
    """A record answers only for its own workload, 16-bit format, fold and
    kernel, and only while the kernel source is the one it was taken on."""
    data = json.load(open(bench.TRAFFIC_FILE))
    recs = data.get("records", [data])
    profiled = {(r["workload"], r["half"], r.get("fold", 1), _kernel_of(r)) for r in recs}
    for half in ("fp16", "bf16"):
        for kernel in KERNELS:
            if ("zero2_7b", half, 1, kernel) not in profiled:
                assert bench.load_traffic("zero2_7b", half, kernel) is None
    assert bench.load_traffic("no_such_workload", "fp16", "adam_kernel") is None
    for rec in recs:
        fold = rec.get("fold", 1)
        got = bench.load_traffic(rec["workload"], rec["half"], _kernel_of(rec), fold)
        if rec["kernel_source_sha256_16"] == bench.kernel_source_hash():
            # counters of the current source: within 0.1 % of the algorithmic bytes (no re-reads)
            assert got == rec["traffic_bytes_per_launch"]
            assert abs(got / rec["algorithmic_bytes_per_launch"] - 1) < 1e-3
            for kernel in KERNELS:
                if (rec["workload"], rec["half"], fold, kernel) not in profiled:
                    assert bench.load_traffic(rec["workload"], rec["half"], kernel, fold) is None
            if (rec["workload"], rec["half"], fold + 7, _kernel_of(rec)) not in profiled:
                assert bench.load_traffic(rec["workload"], rec["half"], _kernel_of(rec), fold + 7) is None
        else:
            assert got is None


def test_more_than_one_gpu_is_refused(capsys):
    with pytest.raises(SystemExit) as e:
        bench.main(["--gpus", "2"])
    assert e.value.code != 0
    assert "one GPU" in capsys.readouterr().err
