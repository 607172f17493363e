"""The chunk plan (bit_adamw_step_amd/csrc/chunk_plan.h: chunk sizing, the re-cut of the last
rounds, dealing chunks to the least-loaded workgroup) built with g++ on the host and run on the
workloads' tensor lists and on seeded random lists: every 128-value unit of every tensor lands
in exactly one chunk, the table is whole rounds of the grid, padding entries are empty, and the
per-workgroup work (in workgroup iterations of 16 units) is balanced to within one chunk."""
import json
import os
import random
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "bit_adamw_step_amd", "csrc")
sys.path.insert(0, ROOT)

DRIVER = r'''
#include <cstdio>
#include <cstdlib>
#include "chunk_plan.h"
using namespace adamw4;
// stdin: G, count, then units per tensor; stdout: one JSON object
int main() {
    unsigned long long G, n;
    if (scanf("%llu %llu", &G, &n) != 2) return 2;
    std::vector<uint64_t> units(n);
    uint64_t total = 0;
    for (auto& u : units) { unsigned long long x; if (scanf("%llu", &x) != 1) return 2; u = x; total += x; }
    const uint32_t cu = pick_chunk_units(total, G);
    std::vector<Chunk> ch;
    for (size_t i = 0; i < n; ++i)
        for (uint64_t u = 0; u < units[i]; u += cu)
            ch.push_back(Chunk{uint32_t(i), uint32_t(u), uint32_t(std::min<uint64_t>(cu, units[i] - u)), 0});
    const size_t before = ch.size();
    balance_chunks(ch, G);
    std::vector<std::vector<unsigned char>> seen(n);
    for (size_t i = 0; i < n; ++i) seen[i].assign(units[i], 0);
    int ok = 1;
    size_t empty = 0;
    uint64_t maxpiece = 0;
    for (const Chunk& c : ch) {
        if (c.units == 0) { ++empty; if (c.tensor || c.first_unit || c.reserved) ok = 0; continue; }
        if (c.tensor >= n || uint64_t(c.first_unit) + c.units > units[c.tensor]) { ok = 0; continue; }
        for (uint64_t u = c.first_unit; u < uint64_t(c.first_unit) + c.units; ++u) seen[c.tensor][u]++;
        maxpiece = std::max<uint64_t>(maxpiece, c.units);
    }
    for (size_t i = 0; i < n; ++i) for (unsigned char v : seen[i]) if (v != 1) ok = 0;
    std::vector<uint64_t> load(G, 0);
    for (size_t c = 0; c < ch.size(); ++c) load[c % G] += (ch[c].units + kPlanRows - 1) / kPlanRows;
    const uint64_t mx = *std::max_element(load.begin(), load.end());
    const uint64_t mn = *std::min_element(load.begin(), load.end());
    printf("{\"ok\": %d, \"cu\": %u, \"before\": %zu, \"after\": %zu, \"empty\": %zu, \"maxpiece\": %llu, "
           "\"maxload\": %llu, \"minload\": %llu}\n", ok, cu, before, ch.size(), empty,
           (unsigned long long)maxpiece, (unsigned long long)mx, (unsigned long long)mn);
    return 0;
}
'''


@pytest.fixture(scope="module")
def plan_exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("chunk_plan")
    src = d / "driver.cpp"
    src.write_text(DRIVER)
    exe = d / "driver"
    subprocess.run([gxx, "-O2", "-std=c++17", "-I", CSRC, "-o", str(exe), str(src)], check=True)
    return str(exe)


def run_plan(exe, G, units):
    inp = f"{G} {len(units)} " + " ".join(str(u) for u in units)
    r = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
    return json.loads(r.stdout)


def units_of(specs):
    """Units per tensor as a step plan walks them: quantized tensors' full blocks only."""
    out = []
    for s in specs:
        quant = s.numel >= 4096 and not (s.flags & 1)
        out.append(s.numel // 128 if quant else (s.numel + 127) // 128)
    return out


def check(res, G):
    assert res["ok"] == 1, res
    if res["before"] > G:
        assert res["after"] % G == 0, res                       # whole rounds
        assert res["maxload"] - res["minload"] <= -(-res["cu"] // 16), res   # within one chunk
    else:
        assert res["after"] == res["before"] and res["empty"] == 0, res


@pytest.mark.parametrize("wname", ["llama2b7", "gpt834m", "gpt130m", "stress", "flat1m"])
@pytest.mark.parametrize("G", [1280, 1024, 768])
def test_workload_lists(plan_exe, wname, G):
    import workloads as W
    res = run_plan(plan_exe, G, units_of(W.WORKLOADS[wname].specs))
    check(res, G)


def test_llama_list_balance(plan_exe):
    """On the 2.7B list at 1280 workgroups (5 per CU): 64-unit chunks, and the most loaded
    workgroup is within 2 iterations (of about 1031) of the least."""
    import workloads as W
    res = run_plan(plan_exe, 1280, units_of(W.WORKLOADS["llama2b7"].specs))
    check(res, 1280)
    assert res["cu"] == 64 and res["maxload"] - res["minload"] <= 2, res


def test_random_lists(plan_exe):
    rng = random.Random(11)
    for _ in range(200):
        G = rng.choice([2, 7, 64, 320, 1024, 1280])
        units = [rng.choice([rng.randint(1, 40), rng.randint(1, 3000), rng.randint(1000, 80000)])
                 for _ in range(rng.randint(1, 50))]
        check(run_plan(plan_exe, G, units), G)
