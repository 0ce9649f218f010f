"""bench.py's command-line contract that needs no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_rotation_sets_are_disjoint_and_cover_the_workload_slots():
    sys.path.insert(0, ROOT)
    import torch
    import bench
    from kda_inputs import make_config
    for index in range(5):
        case = make_config(index)
        base, views = bench.rotation_sets(case, torch)
        sets = [torch.as_strided(base, sh, st, off) for sh, st, off in views]
        flat = torch.cat([s.reshape(-1) for s in sets])
        assert len(set(flat.tolist())) == flat.numel(), index
        assert torch.equal(sets[0], case.slots), index
        for sh, st, off in views:
            assert off + sum((a - 1) * b for a, b in zip(sh, st)) < base.numel()
