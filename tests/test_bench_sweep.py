"""Host logic of bench.py --sweep: one JSON line per workload appended to the
results file, workloads already there skipped, a line cut short ignored."""
import json

import bench


def test_sweep_appends_and_resumes(tmp_path):
    path = str(tmp_path / "sweep.jsonl")
    calls = []

    def run(cid):
        calls.append(cid)
        return {"metric": "m", "value": float(cid), "config": {"workload": f"w{cid}"}}

    assert bench.sweep(path, 3, run) == 0
    assert calls == [0, 1, 2]
    recs = [json.loads(ln) for ln in open(path)]
    assert [r["config_id"] for r in recs] == [0, 1, 2]
    assert [r["value"] for r in recs] == [0.0, 1.0, 2.0]

    # a rerun finds every workload done
    calls.clear()
    bench.sweep(path, 3, run)
    assert calls == []

    # an interrupted run: the last line was cut short, and config 1 is missing
    with open(path, "w") as f:
        f.write(json.dumps({"config_id": 0, "value": 0.0}) + "\n")
        f.write('{"config_id": 2, "val')
    calls.clear()
    bench.sweep(path, 3, run)
    assert calls == [1, 2]
    good = []
    for ln in open(path):
        try:
            good.append(json.loads(ln)["config_id"])
        except ValueError:
            pass
    assert sorted(good) == [0, 1, 2]


def test_sweep_propagates_a_failed_workload(tmp_path):
    path = str(tmp_path / "sweep.jsonl")

    def run(cid):
        if cid == 1:
            raise RuntimeError("bench.py --config 1 exited with 1")
        return {"value": 1.0}

    try:
        bench.sweep(path, 3, run)
    except RuntimeError:
        pass
    else:
        raise AssertionError("the failure must surface")
    assert [json.loads(ln)["config_id"] for ln in open(path)] == [0]
