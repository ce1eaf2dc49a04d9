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


def test_memory_plan_of_the_workloads():
    """The step form and buffers bench.py plans for each workload (no GPU):
    the double-buffered form where it applies, the running sum only where the
    step needs it, the gradient ring and the room left beside the second copy."""
    from synth.workloads import WORKLOADS
    GiB = 1 << 30
    c5, c2, c4, c1 = (WORKLOADS[k] for k in ("zero1_70b", "zero2_7b", "ragged", "tiny"))
    # 8.75e9 elements, K = 1: a 17.5 GB gradient, far beyond the Infinity Cache
    assert bench.double_wanted("auto", 0.0, 1, c5.psi)
    assert not bench.double_wanted("auto", 1.0, 1, c5.psi)              # clipping: in place
    assert not bench.double_wanted("double", 1.0, 1, c5.psi)
    ring = bench.grad_ring(c5.psi, 1, 1, 50, 5, 8)
    assert ring == 2
    assert bench.room_beside_second_copy(c5.psi, 1, 1, ring) == 2 * 2 * c5.psi + 4 * GiB
    assert not bench.needs_running_sum(1, 1, True)
    # the 7B ZeRO-2 shard: its 219 MB gradient stays in the 256 MB cache, so auto keeps the in-place form
    assert not bench.double_wanted("auto", 0.0, 1, c2.psi) and bench.double_wanted("double", 0.0, 1, c2.psi)
    # the tiny workload: its whole state (16.8 MB) fits the cache, the step is launch-bound, one launch wins
    assert bench.double_wanted("auto", 0.0, 1, c1.psi)
    assert not bench.double_wanted("in_place", 0.0, 8, c4.psi)
    # the ragged layout with 8 micro-batches: double-buffered, the sum needed unless all 8 are folded at once
    assert bench.double_wanted("auto", 0.0, 8, c4.psi)
    assert bench.needs_running_sum(8, 1, True) and bench.needs_running_sum(8, 3, True)
    assert not bench.needs_running_sum(8, 8, True) and bench.needs_running_sum(8, 8, False)
    assert bench.grad_ring(c4.psi, 8, 8, 10, 2, 8) == 8 and bench.grad_ring(c4.psi, 8, 1, 10, 2, 8) == 2
    assert bench.room_beside_second_copy(c4.psi, 8, 8, 8) == 8 * 2 * c4.psi + 4 * GiB
    assert bench.room_beside_second_copy(c4.psi, 8, 1, 2) == 2 * 2 * c4.psi + 4 * c4.psi + 4 * GiB
    # small partitions: a 2 GiB ring, capped by the run's draws and the caller's limit
    assert bench.grad_ring(c1.psi, 1, 1, 50, 5, 8) == 8 and bench.grad_ring(c1.psi, 1, 1, 2, 1, 8) == 3
    assert bench.buffers_that_fit(10 * GiB, c5.psi, 2) == 1                # never fewer than one
    assert bench.buffers_that_fit(200 * GiB, c4.psi, 8) == 8
    assert bench.fold_bytes([8]) == 20 and bench.fold_bytes([3, 3, 2]) == 10 + 14 + 12
