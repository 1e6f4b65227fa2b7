"""The no-allocation decode entry point against the workspace decode.

hpkv_paged_attention_decode_noalloc runs the kernels of
hpkv_paged_attention_decode with a fixed scratch array inside the library as
its workspace. Called twice in a row through the C ABI, the second time on a
smaller batch (the scratch then still holds the first call's partials), each
output must equal the workspace decode's bit for bit on the same inputs and
lie within the oracle tolerance (2e-2 absolute for bf16 and f16,
1e-5 + 1e-5 |ref| for f32).
"""
import pytest
import torch

import paged_kv_cache_hpkv_amd as hpkv
import workloads
from paths import decode_errors, host_bits, oracle_step, host_inputs, poison_unused, gpu_step

pytestmark = pytest.mark.gpu


def _run(w):
    t = workloads.make_tensors(w, "cuda")
    poison_unused(w, t)
    h = host_inputs(t)
    _, out_ws = gpu_step(w, t)  # slot mapping + store + the workspace decode
    dev = t.q.device
    out_na = torch.full_like(t.q, float("nan"))
    hpkv.hpkv_paged_attention_decode_noalloc(
        t.q, t.k_cache, t.v_cache, torch.from_numpy(w.block_table).to(dev),
        torch.from_numpy(w.seq_ptr).to(dev), torch.from_numpy(w.context_lens).to(dev), w.scale,
        w.max_context_len, out_na)
    torch.cuda.synchronize()
    assert host_bits(out_na).tobytes() == host_bits(out_ws).tobytes()
    _, _, ref64 = oracle_step(w, h)
    err, ratio, finite = decode_errors(w.dtype, host_bits(out_na), ref64)
    assert finite and ratio <= 1.0, err
    return err


@pytest.mark.parametrize("first,second", [
    (lambda: workloads.gqa(batch=96), lambda: workloads.llama7b(batch=6)),
    (lambda: workloads.qwen3(batch=24), lambda: workloads.tiny(bs=16, dtype="bf16")),
    (lambda: workloads.llama7b(batch=16, dtype="f16"), lambda: workloads.gqa(batch=8,
                                                                             dtype="f16")),
])
def test_noalloc_decode_equals_workspace_decode(first, second):
    w1, w2 = first(), second()
    assert w2.num_seqs < w1.num_seqs
    print(f"[noalloc] {w1.name} then {w2.name}", flush=True)
    e1 = _run(w1)
    e2 = _run(w2)
    print(f"max err {e1:.2e} then {e2:.2e}", flush=True)
