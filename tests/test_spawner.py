"""The session's GPU-free spawner runs programs and returns their status and output."""
import sys


def test_spawner_runs_programs(run_program):
    rc, out, err = run_program([sys.executable, "-c", "import sys; print('hi'); sys.exit(3)"])
    assert rc == 3 and out == "hi\n"
    rc, out, err = run_program(["/nonexistent/program"])
    assert rc == 127 and err
