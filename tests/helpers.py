"""Shared test helpers: device upload of generated inputs, error metric, header parsing."""
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_latent.h")

BF16_TOL = 2e-2  # max |gpu - ref| / max |ref|, bf16 inputs with fp32 accumulation
F32_TOL = 1e-4   # same metric, fp32 inputs


def declared_functions(path: str = HEADER):
    """Names of the functions the C header declares."""
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(mla_[a-z_0-9]+)\s*\(", src,
                                 flags=re.M)))


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    den = np.max(np.abs(ref)) if ref.size else 1.0
    return float(np.max(np.abs(gpu - ref)) / max(den, 1e-30)) if ref.size else 0.0


def tol_for(x) -> float:
    return BF16_TOL if x.is_bf16 else F32_TOL


def check_lse(gpu, refv, tol) -> float:
    """lse: -inf exactly where the oracle has it; elsewhere |gpu - ref| <= tol in absolute terms.
    lse enters every softmax weight as e^{z - lse}, so an absolute error d rescales all weights of
    the row by e^{-d}: the bar is on d itself, not on d relative to the size of lse."""
    gpu = np.asarray(gpu, np.float64)
    refv = np.asarray(refv, np.float64)
    assert gpu.shape == refv.shape, (gpu.shape, refv.shape)
    assert not np.isnan(gpu).any(), "lse holds NaN"
    assert np.array_equal(np.isneginf(gpu), np.isneginf(refv)), "-inf pattern differs"
    fin = np.isfinite(refv)
    err = float(np.max(np.abs(gpu[fin] - refv[fin]))) if fin.any() else 0.0
    assert err <= tol, f"lse abs err {err:.3e} > {tol}"
    return err


def sample_rows(lse_ref, n: int = 48, seed: int = 0, seqs=None):
    """Up to n (b, i, h) rows with a finite oracle lse (a seeded sample, the first and last always in)."""
    lse_ref = np.asarray(lse_ref)
    idx = np.argwhere(np.isfinite(lse_ref))
    if seqs is not None:
        idx = idx[np.isin(idx[:, 0], list(seqs))]
    if len(idx) <= n:
        return [tuple(int(v) for v in r) for r in idx]
    pick = np.random.default_rng(seed).choice(len(idx), n - 2, replace=False)
    pick = np.unique(np.concatenate([[0, len(idx) - 1], pick]))
    return [tuple(int(v) for v in idx[k]) for k in pick]


def check_softmax_mass(q_lat, q_pe, pool, block_table, seq_lens, lse_gpu, rows, *, softmax_scale, tol,
                       causal=True, tree=None) -> float:
    """The oracle recomputes each sampled row's scores and sums e^{z_j - lse_gpu}: the GPU's lse must
    normalise the softmax to one within tol."""
    from oracle import mla_decode as ref
    mass = ref.softmax_mass(q_lat, q_pe, pool, block_table, seq_lens, lse_gpu, rows, softmax_scale=softmax_scale,
                            causal=causal, tree=tree)
    assert not np.isnan(mass).any(), "a sampled row has no keys"
    err = float(np.max(np.abs(mass - 1.0))) if len(rows) else 0.0
    assert err <= tol, f"softmax mass off by {err:.3e} > {tol}"
    return err


def to_device(x, device="cuda"):
    """Upload a DecodeInputs batch (bf16 as bit-exact torch.bfloat16)."""
    import torch

    def conv(a):
        if x.is_bf16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return dict(q_nope=conv(x.q_nope), q_pe=conv(x.q_pe), w_uk=conv(x.w_uk), w_uv=conv(x.w_uv),
                pool=conv(x.pool), block_table=torch.from_numpy(x.block_table).to(device),
                seq_lens=torch.from_numpy(x.seq_lens).to(device))


def device_array(x, dtype_bf16: bool, device="cuda"):
    import torch
    if dtype_bf16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy()


def params_for(x, **kw):
    from deepseek_mla_latent_amd import binding
    w = x.workload
    return binding.make_params(batch=w.batch, q_len=w.q_len, max_seq_len=x.max_seq_len,
                               max_pages_per_seq=x.block_table.shape[1], softmax_scale=w.softmax_scale,
                               causal=kw.get("causal", True),
                               dtype=binding.MLA_BF16 if x.is_bf16 else binding.MLA_F32)
