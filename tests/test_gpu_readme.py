"""The Python example in README.md, run as written, then checked: the pools
bit-exact against the oracle's cache write and the output within the bf16
bar of the oracle's decode."""
import pathlib
import re

import pytest
import torch

import oracle.paged_attention as ref
from paged_kv_cache_19_amd import workloads
from tests.gpu_common import TOL, bits, log

pytestmark = pytest.mark.gpu


def _example() -> str:
    text = (pathlib.Path(__file__).resolve().parents[1] / "README.md").read_text()
    m = re.search(r"```python\n(.*?)```", text, re.S)
    assert m, "README.md holds no python example"
    return m.group(1)


def test_readme_example():
    torch.manual_seed(0)
    ns = {}
    exec(compile(_example(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    B, D = ns["B"], ns["D"]
    bt = ns["block_tables"].cpu()
    lens = ns["seq_lens"].cpu().tolist()
    kc0 = torch.zeros_like(ns["k_cache"], device="cpu")
    vc0 = torch.zeros_like(ns["v_cache"], device="cpu")
    slots = ref.compute_slot_mapping(bt, lens, None, B)
    assert torch.equal(ns["slots"].cpu(), slots), "slots differ from the oracle"
    kc, vc = ref.reshape_and_cache(kc0, vc0, ns["key"].cpu(), ns["value"].cpu(), slots)
    assert torch.equal(bits(ns["k_cache"].cpu()), bits(kc)), "K pool differs from the oracle"
    assert torch.equal(bits(ns["v_cache"].cpu()), bits(vc)), "V pool differs from the oracle"
    expect = ref.decode(ns["query"].cpu(), kc, vc, bt, lens, D ** -0.5)
    err = (ns["out"].cpu().double() - expect).abs().max().item()
    log(f"[readme] example: pools bit-exact, decode_append max-abs err {err:.3e}")
    assert err <= TOL[workloads.BF16]
