"""bench.py's command line on the host: a request for more than one GPU is
refused with a message before anything touches a device.  Called in-process
(no child interpreter is started)."""
import sys

import bench


def test_bench_refuses_more_than_one_gpu(monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert bench.main() == 2
    out = capsys.readouterr()
    assert "one GPU only" in out.err
    assert out.out.strip() == ""
