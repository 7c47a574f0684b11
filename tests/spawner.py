"""Runs commands on behalf of the test process, from a process that never
initialises the GPU.

A process that has initialised the GPU must not exec another program (not even
in a forked child), so GPU programs that a test needs as separate processes are
started from here instead: the test session starts this spawner before anything
touches the GPU and sends it one JSON request per line,
{"cmd": [...], "timeout": seconds}; it answers with one JSON line
{"rc": ..., "stdout": ..., "stderr": ...}.
"""
import json
import os
import subprocess
import sys


def main():
    for line in sys.stdin:
        req = json.loads(line)
        try:
            # the program's own RUNPATH picks its libraries, not an inherited search path
            env = {k: v for k, v in os.environ.items() if k != "LD_LIBRARY_PATH"}
            r = subprocess.run(req["cmd"], capture_output=True, text=True, timeout=req.get("timeout", 120), env=env)
            res = {"rc": r.returncode, "stdout": r.stdout, "stderr": r.stderr}
        except subprocess.TimeoutExpired as e:
            res = {"rc": 124, "stdout": e.stdout or "", "stderr": f"timed out after {e.timeout} s"}
        except OSError as e:
            res = {"rc": 127, "stdout": "", "stderr": str(e)}
        sys.stdout.write(json.dumps(res) + "\n")
        sys.stdout.flush()


if __name__ == "__main__":
    main()
