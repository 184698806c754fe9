"""The library's host state under concurrent callers, checked by ThreadSanitizer (no GPU).

Callers may use the library from several threads (the header promises thread safety for
calls that share no buffers).  The host-side shared state is the tuned-configuration
cache (a mutex), the static workspaces (a mutex) and the per-thread last-error text and
launch recorder.  A driver built with the host pass instrumented runs eight threads
that each replay launch plans (which read the cache), pin and forget configurations
(which write it), query phases and routes, and provoke argument errors, all at once;
ThreadSanitizer must report no data race.  (Positive control, run on the CPU: with the
cache lookup's lock removed, ThreadSanitizer reports the race in the lookup.)
"""
import os
import shutil
import subprocess
import tempfile

import pytest

from conftest import ROOT

import adamw_optimizer_step_muon_amd.build as _build

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "adamw_optimizer_step_muon_amd", "csrc")

DRIVER = r'''
#include <atomic>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>
#include "muon_adamw.h"

static std::atomic<int> failures{0};

static void worker(int id) {
  const std::vector<std::vector<ma_muon_bucket>> lists = {
    {{48, 768, 768}, {12, 768, 3072}, {12, 3072, 768}},
    {{4, 300, 520}, {2, 520, 300}, {3, 96, 96}},
    {{6, 2304, 4096}},
  };
  ma_muon_hparams hp;
  std::memset(&hp, 0, sizeof hp);
  hp.lr = 0.02f; hp.momentum = 0.95f; hp.ns_eps = 1e-7f; hp.nesterov = 1; hp.ns_steps = 3;
  for (int it = 0; it < 6; ++it) {
    const auto& l = lists[(id + it) % lists.size()];
    hp.ns_mode = (id + it) & 1;
    ma_plan_report rep;
    if (ma_muon_check_plan(l.data(), (int)l.size(), &hp, 0, &rep) != MA_OK) ++failures;
    const int nph = ma_muon_phases(l.data(), (int)l.size(), &hp, nullptr);
    if (nph < 1) { ++failures; continue; }
    std::vector<ma_gemm_config> cfg(3 * nph, ma_gemm_config{0, 2 + (id % 3), -1, 0, 1 + (id & 1)});
    if (ma_muon_tune_configs(l.data(), (int)l.size(), &hp, nullptr, 0, nullptr, 0, cfg.data()) != MA_OK)
      ++failures;
    if (ma_muon_check_plan(l.data(), (int)l.size(), &hp, 0, &rep) != MA_OK) ++failures;
    if (it % 3 == 2) ma_muon_tune_reset();
    ma_muon_route r;
    if (ma_muon_route_of(l[0].A, l[0].B, &hp, &r) != MA_OK) ++failures;
    // an argument error: its text stays with this thread
    if (ma_muon_phases(l.data(), -1 - id, &hp, nullptr) != MA_ERR_INVALID_ARG) ++failures;
    char want[32];
    std::snprintf(want, sizeof want, "n_buckets %d", -1 - id);
    if (!std::strstr(ma_last_error(), want)) ++failures;
  }
}

int main() {
  std::vector<std::thread> ts;
  for (int i = 0; i < 8; ++i) ts.emplace_back(worker, i);
  for (auto& t : ts) t.join();
  std::printf("threads done, %d failures\n", failures.load());
  return failures.load() ? 1 : 0;
}
'''


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_state_under_thread_sanitizer():
    tmp = tempfile.mkdtemp(prefix="ma_tsan_")
    try:
        drv = os.path.join(tmp, "driver.cpp")
        with open(drv, "w") as f:
            f.write(DRIVER)
        exe = os.path.join(tmp, "driver")
        flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-pthread",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-Xarch_host", "-fsanitize=thread", "-I", os.path.join(ROOT, "include")]
        srcs = [os.path.join(CSRC, s) for s in _build.SOURCES]
        r = subprocess.run([HIPCC, *flags, *srcs, drv, "-o", exe], capture_output=True,
                           text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, TSAN_OPTIONS="halt_on_error=0:report_signal_unsafe=0")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
        out = r.stdout + r.stderr
        assert "ThreadSanitizer" not in out, out[-5000:]
        assert r.returncode == 0 and "0 failures" in out, out[-4000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
