"""The commands recorded in profiles/ name kbench cases, workloads and
bench.py options that still exist, so each summary can be re-made from the
committed sources."""
import glob
import os
import re

import q3synth
from decoder_only_qwen3_amd import kbench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _commands():
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if "rocprofv3" in line and " -- " in line:
                yield os.path.basename(path), line.strip()


def test_every_profile_records_a_command():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert paths
    with_cmd = {p for p, _ in _commands()}
    assert with_cmd == {os.path.basename(p) for p in paths}


def test_profile_commands_name_existing_cases_and_workloads():
    bench_src = open(os.path.join(ROOT, "bench.py")).read()
    for path, cmd in _commands():
        for names in re.findall(r"--kernels (\S+)", cmd):
            for k in names.split(","):
                assert k in kbench.CASES, (path, k)
        for w in re.findall(r"--workload (\S+)", cmd):
            assert w in q3synth.WORKLOADS, (path, w)
        if "bench.py" in cmd:
            for opt in re.findall(r"(--[a-z][a-z0-9-]*)", cmd.split("bench.py", 1)[1]):
                assert f'"{opt}"' in bench_src, (path, opt)
