"""Helpers for the GPU parity tests: host storage arrays <-> device tensors, running the HIP
path through the package, and the error gates. Not a test module."""
import numpy as np
import torch

from oracle import paged_attention as oracle_pa

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# Max-abs-error gates against the fp64 oracle for fp32 output (the pages fix none; these
# are the stated targets): 1e-5 for fp32 KV, 2e-3 for 16-bit KV.
GATE = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def run_decode(case, out_dtype=None, partition_size=512, q=None, k=None, v=None, tables=None,
               lens=None, scale=None):
    """Runs the HIP decode on a PagedDecodeCase (host arrays uploaded unless device tensors
    are given). Returns the output as float64 numpy."""
    import paged_kv_cache_402_amd as pk
    dt = case.dtype
    q = to_dev(case.q, dt) if q is None else q
    k = to_dev(case.k_cache, dt) if k is None else k
    v = to_dev(case.v_cache, dt) if v is None else v
    tables = i32(case.block_tables) if tables is None else tables
    lens = i32(case.seq_lens) if lens is None else lens
    odt = torch.float32 if out_dtype is None else TORCH_DT[out_dtype]
    out = torch.full(tuple(q.shape), float("nan"), dtype=odt, device=q.device)
    pk.paged_attention_decode(out, q, k, v, tables, lens, case.scale if scale is None else scale,
                              partition_size=partition_size)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), out


def oracle(case, seqs=None):
    return oracle_pa.decode_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                                      case.seq_lens, case.scale, case.dtype, seqs=seqs)


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of |x| in a 16-bit output format (rounding of the output)."""
    ax = np.maximum(np.abs(x), 1e-30)
    mant = {"bf16": 8, "f16": 11}[dtype]
    e = np.floor(np.log2(ax))
    if dtype == "f16":
        e = np.maximum(e, -14)
    return 2.0 ** (e - mant)


def out_gate(ref: np.ndarray, kv_dtype: str, out_dtype) -> np.ndarray:
    """Per-element max-abs-error gate for an output of out_dtype (None or "f32": fp32).

    fp32 output: GATE[kv_dtype]. A 16-bit output is the fp32 result rounded once, to nearest,
    which alone can move it by half an ulp: 1.95e-3 for bf16 |x| in [0.5, 1) and 3.9e-3 in
    [1, 2). The gate is max(GATE[kv_dtype], half_ulp(|ref|) + 1e-5): the 2e-3 bar of 16-bit KV
    wherever one rounding fits inside it (bf16 |x| < 1, fp16 |x| < 8), and otherwise half an
    ulp plus the 1e-5 that the fp32 arithmetic before the rounding is held to (its fp32-KV
    bar), so a value that lands next to a rounding midpoint still passes while a second
    rounding or a wrong digit does not. Never looser than 2e-3."""
    if out_dtype is None or out_dtype == "f32":
        return np.full(np.shape(ref), GATE[kv_dtype])
    return np.maximum(GATE[kv_dtype], half_ulp(ref, out_dtype) + GATE["f32"])


def max_err(got, ref, rows=None):
    if rows is not None:
        got, ref = got[rows], ref[rows]
    return float(np.max(np.abs(got - ref))) if got.size else 0.0
