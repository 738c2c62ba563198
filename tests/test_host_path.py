"""The host side of a call without a GPU: what a call costs before its first
launch (argument checks, device query, cached plan), the plan cache and the
CU count the plans are made for.

With no device visible a valid call stops right before the launch and returns
GEMM_ERR_HIP, so timing it measures everything the library does on the host
per call except the launch itself. A small C program does the timing
(dlopen + clock_gettime), so no Python overhead is counted.
"""
import os
import subprocess

import pytest

from dense_fp16_gemm_03_amd import gemm, inputs

HARNESS = r"""
#include <dlfcn.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <time.h>
typedef int (*fn_t)(int64_t, int64_t, int64_t, const void*, int64_t, const void*, int64_t,
                    float*, int64_t, void*);
static double now_ns(void) {
  struct timespec t;
  clock_gettime(CLOCK_MONOTONIC, &t);
  return t.tv_sec * 1e9 + t.tv_nsec;
}
int main(int argc, char** argv) {
  void* h = dlopen(argv[1], RTLD_NOW);
  if (!h) { fprintf(stderr, "%s\n", dlerror()); return 2; }
  fn_t f = (fn_t)dlsym(h, "gemm_f16_f32_abt");
  const int64_t M = atoll(argv[2]), N = atoll(argv[3]), K = atoll(argv[4]);
  const int iters = atoi(argv[5]);
  const char* A = (const char*)0x100000000ull;
  const char* B = (const char*)0x200000000ull;
  float* C = (float*)0x400000000ull;
  double t0 = now_ns();
  int st = f(M, N, K, A, K, B, K, C, N, 0);
  double t1 = now_ns();
  for (int i = 0; i < iters; ++i) st |= f(M, N, K, A, K, B, K, C, N, 0) << 8;
  double t2 = now_ns();
  printf("%d %.1f %.1f\n", st, t1 - t0, (t2 - t1) / iters);
  return 0;
}
"""


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    d = tmp_path_factory.mktemp("host_path")
    src, exe = d / "harness.c", d / "harness"
    src.write_text(HARNESS)
    subprocess.run(["gcc", "-O2", str(src), "-o", str(exe), "-ldl"], check=True)
    return str(exe)


def _no_device():
    try:
        import torch

        return not torch.cuda.is_available()
    except ImportError:
        return True


@pytest.mark.skipif(not _no_device(), reason="measures the host path where no device is visible")
@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_host_cost_per_call(harness, name):
    """Argument checks, device query and the cached plan: a few hundred
    nanoseconds a call after the first (the figure is printed)."""
    M, N, K = inputs.WORKLOADS[name]
    out = subprocess.run([harness, gemm.LIBRARY, str(M), str(N), str(K), "20000"],
                         capture_output=True, text=True, timeout=120, check=True).stdout.split()
    status, first_ns, per_call_ns = int(out[0]), float(out[1]), float(out[2])
    print(f"{name}: first call {first_ns / 1e3:.1f} us, then {per_call_ns:.0f} ns a call "
          "(checks + device query + cached plan)")
    assert status == 3 | (3 << 8)  # GEMM_ERR_HIP: no device to launch on
    assert per_call_ns < 20000


def test_plan_cache_follows_the_override():
    """Cached plans never outlive an override change: the same shape plans
    differently under an override and returns to the default rule after it."""
    M, N, K = inputs.WORKLOADS["1024x1024x65536"]
    default = gemm.gemm_f16_f32_abt_describe(M, N, K)
    assert "splits=16" in default
    gemm.gemm_f16_set_plan_override("kid=35,splits=8")
    forced = gemm.gemm_f16_f32_abt_describe(M, N, K)
    assert "kid=35" in forced and "splits=8" in forced
    gemm.gemm_f16_set_plan_override("")
    assert gemm.gemm_f16_f32_abt_describe(M, N, K) == default


def test_workspace_size_and_caller_check_share_the_cu_count():
    """On a device with fewer CUs (planned here for 32 through the override)
    the split is smaller, and the workspace size and the check a _ws call
    makes use the same plan: the reported size passes the check (the call
    then stops at the missing device, GEMM_ERR_HIP), a byte less fails it
    (GEMM_ERR_WORKSPACE)."""
    M, N, K = inputs.WORKLOADS["1024x1024x65536"]
    A, B, C, W = 0x10000000, 0x20000000, 0x30000000, 0x40000000
    full = gemm.gemm_f16_f32_abt_workspace_size(M, N, K)
    assert full == 16 * 16 * 256 * 256 * 4  # 16 tiles x 16 shares on 256 CUs
    gemm.gemm_f16_set_plan_override("cus=32")
    need = gemm.gemm_f16_f32_abt_workspace_size(M, N, K)
    assert need == 16 * 2 * 256 * 256 * 4  # 2 shares a tile fill 32 CUs
    assert "splits=2" in gemm.gemm_f16_f32_abt_describe(M, N, K)
    expect_ok = 3 if _no_device() else 0
    if _no_device():
        assert gemm.gemm_f16_f32_abt_ws(M, N, K, A, K, B, K, C, N, W, need, 0) == expect_ok
    assert gemm.gemm_f16_f32_abt_ws(M, N, K, A, K, B, K, C, N, W, need - 1, 0) == 5
    gemm.gemm_f16_set_plan_override("")
    assert gemm.gemm_f16_f32_abt_workspace_size(M, N, K) == full
