"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

import oracle as O
import qmoe_synth as S

# Float parity bar, applied to the pre-rounding fp32 output: max-abs error at
# most 1e-2 * RMS of the exact output.  The bf16 output may differ by that
# plus half a bf16 ulp of the exact value (its own rounding).
REL_TOL = 1e-2
# Top-k: ids must match exactly unless the exact scores at ranks k and k+1
# are closer than this (fp32 accumulation of a 2816-term dot product of
# ~1e-2-sized terms is good to ~1e-6); then the GPU's choice must be valid.
NEAR_TIE = 1e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def run_gpu(M, dev, x_bits, path="auto", ws=None, **kw):
    """One call with fp32 output and one with bf16 output; routing captured.
    Extra keywords go to both calls."""
    x = bf16_tensor(x_bits)
    T = x.shape[0]
    ids = torch.empty((T, dev.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, dev.top_k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, dev.num_experts), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = dev.new_workspace(T)
    o32 = M.moe_layer_forward(dev, x, workspace=ws, path=path, out_dtype=torch.float32, topk_ids=ids, topk_w=w,
                              logits=lg, **kw)
    o16 = M.moe_layer_forward(dev, x, workspace=ws, path=path, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert M.workspace_errors(ws) == 0, "a bounded wait of the single-launch path gave up"
    return dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), logits=lg.cpu().numpy(),
                out32=o32.cpu().numpy().astype(np.float64), out16=bf16_bits(o16))


def check_routing(ref, got, k):
    """ids exact (or a valid choice at an exact near-tie); weights to 1e-5."""
    excused = 0
    for t in range(ref["ids"].shape[0]):
        if np.array_equal(ref["ids"][t], got["ids"][t]):
            continue
        srt = np.sort(ref["logits"][t])[::-1]
        gap = srt[k - 1] - srt[k]
        assert gap < NEAR_TIE, "token %d: ids %s vs oracle %s (gap %.3g)" % (t, got["ids"][t], ref["ids"][t], gap)
        assert np.all(ref["logits"][t][got["ids"][t]] >= srt[k - 1] - NEAR_TIE)
        excused += 1
    ok = np.all(ref["ids"] == got["ids"], axis=1)
    assert np.allclose(got["w"][ok], ref["w"][ok], rtol=0, atol=1e-5)
    assert np.allclose(got["logits"], ref["logits"], rtol=0, atol=1e-4)
    return ok, excused


def check_output(ref, got, ok_rows=None, rel_tol=REL_TOL):
    rows = slice(None) if ok_rows is None else ok_rows
    r64 = ref["out64"][rows]
    rms = np.sqrt(np.mean(r64 ** 2))
    err32 = np.max(np.abs(got["out32"][rows] - r64)) if r64.size else 0.0
    assert err32 <= rel_tol * rms, "fp32 output error %.3g > %.3g * RMS %.3g" % (err32, rel_tol, rms)
    o16 = bf16_to_f64(got["out16"][rows])
    assert np.all(np.abs(o16 - r64) <= rel_tol * rms + bf16_half_ulp(r64) * 1.0001)
    # the bf16 output is the fp32 output rounded once
    want16 = torch.from_numpy(got["out32"][rows].astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(bf16_bits(want16), got["out16"][rows])
    return err32 / max(rms, 1e-300)
