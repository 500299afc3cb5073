"""The library's host code built alone with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer (no HIP): the shared LRU policy with miss splits,
resizes and injected fill failures (a mock copier), and the CPU expert kernel,
each compared with the oracle. Any sanitizer report fails the run.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch
import dataclasses

import oracle
from tests.blob_layout import bf16_bits, bf16_blob
from tests.parity import check_close
from workloads import gen
from workloads.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routed_expert_layer_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def host_check(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("host") / "host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g"] + SAN + [
        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-mavx512f", "-mavx512bw", "-mavx512vl", "-mavx512bf16",
        os.path.join(ROOT, "tests", "native", "host_check.cpp"), os.path.join(CSRC, "lru_policy.cpp"),
        os.path.join(CSRC, "cpu_expert.cpp"), "-o", out, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def run(exe, commands):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], input="\n".join(commands) + "\n", capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout.splitlines()


def scenario(S, E, L, steps, max_active, seed, split=None, fail_p=0.0, resize_at=None):
    """Commands for the native driver and the lines the oracle expects from them."""
    r = np.random.default_rng(seed)
    sim = oracle.SharedLRU(S)
    cmds, want = [f"cache {L * E} {S}"], []
    if split:
        cmds.append(f"split {split[0]} {split[1]}")
        sim.set_split(*split)
    fail_in = -1  # copies left before the failing one
    for step in range(steps):
        if resize_at and step == resize_at[0]:
            cmds.append(f"resize {resize_at[1]}")
            want += [f"move {k} {a} {b}" for k, a, b in sim.resize(resize_at[1])]
        for layer in range(L):
            if fail_in < 0 and r.random() < fail_p:
                fail_in = int(r.integers(0, 4))
                cmds.append(f"fail {fail_in}")
            n = int(r.integers(1, max_active + 1))
            experts = sorted(r.choice(E, size=n, replace=False).tolist())
            cmds.append(f"step {step} {layer} {E} {n} " + " ".join(map(str, experts)))
            _, recs = sim.resolve(step, layer, E, experts)
            want += [f"rec {c.step} {c.layer} {c.key} {c.hit} {c.slot} {c.victim} {c.wave}" for c in recs]
            gpu_misses = [c for c in recs if not c.hit and c.slot >= 0]
            for w in range(max((c.wave for c in recs), default=-1) + 1):
                batch = [c.key for c in gpu_misses if c.wave == w]
                failed = None
                for j in range(len(batch)):
                    if fail_in >= 0:
                        fail_in -= 1
                        if fail_in < 0:
                            failed = j
                            break
                if failed is None:
                    continue
                # the failed copy's key and the later ones of its batch end unmapped (a key that a later
                # wave's miss already evicted in the resolve is unmapped anyway)
                for key in batch[failed:]:
                    sim.drop(key)
                    want.append(f"drop {key}")
                for c in gpu_misses:
                    if c.wave > w and sim.drop(c.key):
                        want.append(f"drop {c.key}")
                break
        if step % 7 == 0 or fail_p:
            cmds.append("table")
            want += [f"res {k} {sim.key_slot[k]}" for k in sorted(sim.key_slot)]
    return cmds, want


@pytest.mark.parametrize("S,E,L,max_active,split,fail_p,resize_at", [
    (8, 16, 1, 14, None, 0.0, None),          # waves (working sets above S)
    (8, 16, 1, 14, None, 0.25, None),         # waves with failed fills
    (16, 32, 4, 10, (3, 2), 0.15, None),      # miss split and failures
    (12, 24, 3, 8, None, 0.1, (20, 5)),       # shrink after failures
    (4, 20, 2, 6, (1, 4), 0.2, (15, 9)),      # grow, split, failures
])
def test_policy_under_sanitizers_matches_oracle(host_check, S, E, L, max_active, split, fail_p, resize_at):
    cmds, want = scenario(S, E, L, 40, max_active, seed=S * 7 + E, split=split, fail_p=fail_p,
                          resize_at=resize_at)
    got = run(host_check, cmds)
    assert got == want
    if fail_p:
        assert any(w.startswith("drop") for w in want)


@pytest.mark.parametrize("H,I,rows,threads", [(256, 128, 3, 1), (512, 384, 8, 4), (1024, 256, 16, 3)])
def test_cpu_ffn_under_sanitizers_matches_oracle(host_check, tmp_path, H, I, rows, threads):
    cfg = dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name=f"san{H}x{I}", H=H, I=I)
    W1, W3, W2 = gen.expert_weights(cfg, 0, 2)
    x = gen.normal((rows, H), 1.0, ("san-x", H, I, rows), dtype=torch.bfloat16)
    bf16_blob(W1, W3, W2).tofile(tmp_path / "blob")
    bf16_bits(x).tofile(tmp_path / "x")
    got = run(host_check, [f"ffn {tmp_path / 'blob'} {tmp_path / 'x'} {tmp_path / 'y'} {H} {I} {rows} {threads}"])
    assert got == ["ffn 0"]
    y = np.fromfile(tmp_path / "y", np.float32).reshape(rows, H)
    ref = oracle.swiglu_expert(x.float().numpy(), W1.float().numpy(), W3.float().numpy(), W2.float().numpy())
    check_close(y, ref, f"sanitized cpu ffn H{H} I{I} rows{rows}")
