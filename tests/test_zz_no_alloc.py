"""The allocation-free decode entry point (pkv_paged_attention_decode_noalloc) through the C
ABI, against pkv_paged_attention_decode with a caller workspace and against the fp64 oracle
(MI355X only). Two calls in a row share the library's static scratch area; the second is
smaller and must not see the first call's partials."""
import ctypes

import numpy as np
import pytest
import torch

from workloads import gen
from tests.gpu_util import GATE, i32, max_err, oracle, out_gate, to_dev

pytestmark = pytest.mark.gpu

KV = {"f32": 0, "f16": 1, "bf16": 2}
STATIC_BYTES = 64 << 20


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_402_amd  # noqa: F401


def _lib():
    from paged_kv_cache_402_amd import _lib
    return _lib


def _args(case, out, q, k, v, tables, lens, part):
    B, Hq, D = q.shape
    return (out.data_ptr(), KV[case.dtype] if out.dtype != torch.float32 else 0, q.data_ptr(),
            k.data_ptr(), v.data_ptr(), KV[case.dtype], tables.data_ptr(), lens.data_ptr(), B,
            Hq, case.num_kv_heads, D, case.block_size, case.num_blocks,
            case.block_tables.shape[1], ctypes.c_float(case.scale), part)


def _both(case, part, out_dtype, policy):
    """(no-alloc output, workspace output) as float64 host arrays; policy: the KV read
    cache policy both calls take."""
    L = _lib()
    dt = case.dtype
    q, k, v = to_dev(case.q, dt), to_dev(case.k_cache, dt), to_dev(case.v_cache, dt)
    tables, lens = i32(case.block_tables), i32(case.seq_lens)
    B, Hq, D = q.shape
    odt = torch.float32 if out_dtype == "f32" else q.dtype
    out_na = torch.full((B, Hq, D), float("nan"), dtype=odt, device="cuda")
    out_ws = torch.full_like(out_na, float("nan"))
    stream = torch.cuda.current_stream().cuda_stream
    st = L.lib.pkv_paged_attention_decode_noalloc(*_args(case, out_na, q, k, v, tables, lens,
                                                         part), policy, stream)
    assert st == 0, L.last_error()
    need = L.lib.pkv_decode_workspace_bytes(B, Hq, case.block_tables.shape[1], case.block_size,
                                            D, part)
    assert 0 < need <= STATIC_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = L.lib.pkv_paged_attention_decode(*_args(case, out_ws, q, k, v, tables, lens, part),
                                          ws.data_ptr(), need, policy, stream)
    assert st == 0, L.last_error()
    torch.cuda.synchronize()
    return (out_na.float().cpu().numpy().astype(np.float64),
            out_ws.float().cpu().numpy().astype(np.float64))


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    rng = np.random.default_rng(7100)
    big = gen.make_case("na1", rng, [int(x) for x in rng.integers(1, 3000, size=24)] + [3000, 1],
                        32, 8, 128, 16, "bf16")
    got, want = _both(big, 512, "f32", 0)
    assert np.array_equal(got, want)              # same kernels, same partitions: bitwise
    assert max_err(got, oracle(big)) <= GATE["bf16"]
    # a smaller batch next: the static area still holds the first call's partials
    rng = np.random.default_rng(7101)
    small = gen.make_case("na2", rng, [700, 33, 1500, 512, 0], 8, 8, 64, 32, "f16")
    got, want = _both(small, 256, "f16", 1)
    assert np.array_equal(got, want)
    ref = oracle(small)
    assert (np.abs(got - ref) <= out_gate(ref, "f16", "f16")).all()


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """Partials above 64 MiB: PKV_EWORKSPACE on the host, nothing launched (out untouched)."""
    L = _lib()
    B, Hq, Hkv, D, bs, W = 64, 64, 8, 128, 64, 2048    # 131072-token tables at 512: 262 MiB
    need = L.lib.pkv_decode_workspace_bytes(B, Hq, W, bs, D, 512)
    assert need > STATIC_BYTES
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((8, Hkv, bs, D), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, Hq, D), 7.0, dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros((B, W), dtype=torch.int32, device="cuda")
    lens = torch.full((B,), 100, dtype=torch.int32, device="cuda")
    st = L.lib.pkv_paged_attention_decode_noalloc(
        out.data_ptr(), 2, q.data_ptr(), k.data_ptr(), k.data_ptr(), 2, tables.data_ptr(),
        lens.data_ptr(), B, Hq, Hkv, D, bs, 8, W, ctypes.c_float(0.1), 512, 0,
        torch.cuda.current_stream().cuda_stream)
    assert st == -6 and "static area" in L.last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
