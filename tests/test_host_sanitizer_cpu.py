"""The library's host code under AddressSanitizer (no GPU needed).

The four sources are compiled again with the host pass instrumented (the device code is
not) and linked into a small driver that walks every host-only path a caller can reach
without a GPU: routing, phases, workspace sizing, the launch-plan dry run of every
workload's step in both iteration modes (which runs the whole planning and launch
sequence through the recording launchers), configuration pins and their rejections, and
the argument checks of every entry point that rejects before launching.  Any heap or
stack error fails the test.  (A positive control was run on the CPU: a driver passing a
two-entry array to ma_muon_phases for three buckets is stopped by AddressSanitizer inside
the library's host code.)
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

from conftest import ROOT

import adamw_optimizer_step_muon_amd.build as _build

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "adamw_optimizer_step_muon_amd", "csrc")

DRIVER = r'''
#include <cstdio>
#include <cstring>
#include <vector>
#include "muon_adamw.h"

static int failures = 0;
#define EXPECT(c) do { if (!(c)) { std::printf("FAILED %s:%d %s\n", __FILE__, __LINE__, #c); ++failures; } } while (0)

static ma_muon_hparams hp_of(int mode, int steps) {
  ma_muon_hparams hp;
  std::memset(&hp, 0, sizeof hp);
  hp.lr = 0.02f; hp.momentum = 0.95f; hp.weight_decay = 0.1f; hp.ns_eps = 1e-7f;
  hp.nesterov = 1; hp.ns_steps = steps; hp.ns_mode = mode;
  return hp;
}

int main() {
  const std::vector<std::vector<ma_muon_bucket>> lists = {
    {{1, 64, 128}, {1, 128, 64}},
    {{48, 768, 768}, {12, 768, 3072}, {12, 3072, 768}},
    {{80, 1280, 1280}, {20, 1280, 5120}, {20, 5120, 1280}},
    {{48, 2048, 2048}, {48, 2048, 512}, {24, 2048, 8192}, {24, 8192, 2048}},
    {{8, 8192, 28672}, {8, 28672, 8192}, {16, 8192, 8192}},
    {{3, 300, 520}, {2, 520, 300}, {1, 257, 129}, {4, 96, 96}, {2, 1, 7}, {0, 5, 5}},
  };
  for (const auto& l : lists) {
    for (int mode = 0; mode < 2; ++mode)
      for (int steps : {0, 1, 5, 9}) {
        ma_muon_hparams hp = hp_of(mode, steps);
        ma_plan_report rep;
        EXPECT(ma_muon_check_plan(l.data(), (int)l.size(), &hp, 0, &rep) == MA_OK);
        EXPECT(ma_muon_check_plan(l.data(), 1, &hp, 1, &rep) == MA_OK || l[0].K == 0);
        std::vector<int32_t> phase_of(l.size());
        const int32_t nph = ma_muon_phases(l.data(), (int)l.size(), &hp, phase_of.data());
        EXPECT(nph >= 1);
        EXPECT(ma_muon_workspace_bytes(l.data(), (int)l.size(), &hp) > 0);
        // pin every product to 128 then to the defaults (both accepted on every phase)
        std::vector<int32_t> tiles(3 * nph, 128);
        ma_muon_tune(l.data(), (int)l.size(), &hp, nullptr, 0, nullptr, 0, tiles.data());
        EXPECT(ma_muon_check_plan(l.data(), (int)l.size(), &hp, 0, &rep) == MA_OK);
        std::vector<ma_gemm_config> cfg(3 * nph, ma_gemm_config{0, 8, -1, 0, 2});
        EXPECT(ma_muon_tune_configs(l.data(), (int)l.size(), &hp, nullptr, 0, nullptr, 0,
                                    cfg.data()) == MA_OK);
        EXPECT(ma_muon_check_plan(l.data(), (int)l.size(), &hp, 0, &rep) == MA_OK);
        cfg.assign(3 * nph, ma_gemm_config{0, 0, -1, 7, 0});
        EXPECT(ma_muon_tune_configs(l.data(), (int)l.size(), &hp, nullptr, 0, nullptr, 0,
                                    cfg.data()) == MA_ERR_INVALID_ARG);
        ma_muon_tune_reset();
      }
    for (const auto& b : l) {
      ma_muon_route r;
      if (b.K > 0) EXPECT(ma_muon_route_of(b.A, b.B, nullptr, &r) == MA_OK);
    }
  }
  // rejections before any launch
  ma_muon_hparams hp = hp_of(0, 5);
  ma_muon_bucket bad[2] = {{2, 64, 64, (float*)0x1000, (const float*)0x100000, (float*)0x200000},
                           {2, 64, 64, (float*)0x1000, (const float*)0x300000, (float*)0x400000}};
  EXPECT(ma_muon_step(bad, 2, &hp, nullptr, 0, nullptr, nullptr) == MA_ERR_INVALID_ARG);
  EXPECT(ma_muon_step_static(bad, 2, &hp, nullptr, nullptr) == MA_ERR_INVALID_ARG);
  EXPECT(ma_muon_step(bad, -1, &hp, nullptr, 0, nullptr, nullptr) == MA_ERR_INVALID_ARG);
  hp.ns_steps = 65;
  EXPECT(ma_muon_step(bad, 1, &hp, nullptr, 0, nullptr, nullptr) == MA_ERR_INVALID_ARG);
  ma_adamw_hparams ah = {1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 0, 1, 0};
  EXPECT(ma_adamw_step((float*)0x1000, (const float*)0x2000, (float*)0x3000, (float*)0x4000, 16,
                       &ah, nullptr) == MA_ERR_INVALID_ARG);  // step 0
  std::vector<ma_adamw_segment> segs(100);
  for (int i = 0; i < 100; ++i)
    segs[i] = ma_adamw_segment{(float*)(uintptr_t)(0x100000 * (4 * i + 1)),
                               (const float*)(uintptr_t)(0x100000 * (4 * i + 2)),
                               (float*)(uintptr_t)(0x100000 * (4 * i + 3)),
                               (float*)(uintptr_t)(0x100000 * (4 * i + 4)), 1000};
  segs[77].exp_avg = segs[3].param;  // overlap between segments
  ah.step = 1;
  EXPECT(ma_adamw_step_multi(segs.data(), 100, &ah, nullptr) == MA_ERR_INVALID_ARG);
  const float* in[4] = {(const float*)0x10000, (const float*)0x20008, nullptr, nullptr};
  float* out[3] = {(float*)0x30000, nullptr, nullptr};
  EXPECT(ma_stream_probe(in, 2, out, 1, 4096, nullptr) == MA_ERR_INVALID_ARG);  // misaligned
  EXPECT(std::strlen(ma_last_error()) > 0);
  EXPECT(std::strcmp(ma_status_string(MA_ERR_INTERNAL), "internal check failed") == 0);
  std::printf("host paths done, %d failures\n", failures);
  return failures ? 1 : 0;
}
'''


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_code_under_address_sanitizer():
    tmp = tempfile.mkdtemp(prefix="ma_asan_")
    try:
        drv = os.path.join(tmp, "driver.cpp")
        with open(drv, "w") as f:
            f.write(DRIVER)
        exe = os.path.join(tmp, "driver")
        flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-I", os.path.join(ROOT, "include")]
        srcs = [os.path.join(CSRC, s) for s in _build.SOURCES]
        r = subprocess.run([HIPCC, *flags, *srcs, drv, "-o", exe], capture_output=True,
                           text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
        out = r.stdout + r.stderr
        assert "AddressSanitizer" not in out, out[-4000:]
        assert r.returncode == 0 and "0 failures" in out, out[-4000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
