"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws numbers and rounds them to the storage type; it holds
none of the codec's arithmetic, so the CPU oracle and the GPU library can both
be fed from it.  The pages measure real checkpoints (Llama 3.1, Falcon-7B,
Mistral, ... in THEORY-599's summary of ZipNN Table II and Fig. 2) and real K/V
caches; none are available here, so Gaussian stand-ins of the same shapes and
scales take their place.

Recipe (every tensor has its own torch.Generator seeded with seed*1000 + i):
  * draws are float64 standard normals, scaled in float64, rounded once to
    float32 (round-to-nearest-even), and from there to the storage type;
  * BF16 storage: float32 -> bfloat16 by torch's cast (round-to-nearest-even);
  * FP32 "clean": the regular float32 with its low 16 fraction bits cleared;
  * FP8 E4M3: per 128-element block scaled so max|z| maps to 448, clamped to
    +-448 and cast to float8_e4m3fn (round-to-nearest-even, no NaN produced);
  * FP4 E2M1 pairs: per 32-value block scaled so max|z| maps to 6 (the
    largest E2M1 magnitude), rounded to the nearest E2M1 value (ties to the
    even code), two values per byte, the first in the low nibble;
  * perturbed copy of a BF16 weight: bf16(fp32(w) + N(0, 1e-4)).
Host (cpu) and device (cuda) generators produce different streams; tests that
compare the two sides always generate once and copy.
"""
from __future__ import annotations

import torch

GEN_BLOCK = 1 << 26  # elements drawn per call, bounds float64 temporaries


def _gen(device, seed: int, i: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + i)
    return g


def gaussian(n: int, mean: float, std: float, out_dtype, device="cpu", seed=0, i=0):
    """float64 N(mean, std) rounded to float32, then cast to out_dtype."""
    g = _gen(device, seed, i)
    out = torch.empty(n, dtype=out_dtype, device=device)
    for s in range(0, n, GEN_BLOCK):
        m = min(GEN_BLOCK, n - s)
        z = torch.randn(m, dtype=torch.float64, device=device, generator=g)
        out[s:s + m] = (z * std + mean).to(torch.float32).to(out_dtype)
    return out


def uniform_sigma(lo: float, hi: float, seed: int, i: int) -> float:
    g = _gen("cpu", seed, 100000 + i)
    return float(lo + (hi - lo) * torch.rand(1, dtype=torch.float64, generator=g).item())


def bits(t: torch.Tensor) -> torch.Tensor:
    """The same storage viewed as unsigned bit patterns."""
    return t.view({2: torch.uint16, 4: torch.uint32, 1: torch.uint8}[t.element_size()])


# ------------------------------------------------------------------ configs --
def single_bf16(n=1 << 20, std=0.02, device="cpu", seed=1):
    """Single BF16 tensor of 2^20 elements from N(0, 0.02)."""
    return [("w", gaussian(n, 0.0, std, torch.bfloat16, device, seed, 0))]


def block_shapes(hidden=4096, kv=1024, ffn=14336):
    """One Llama-style 8B transformer block, in storage order."""
    return [("attn_norm", (hidden,)), ("wq", (hidden, hidden)), ("wk", (kv, hidden)),
            ("wv", (kv, hidden)), ("wo", (hidden, hidden)), ("ffn_norm", (hidden,)),
            ("w_gate", (ffn, hidden)), ("w_up", (ffn, hidden)), ("w_down", (hidden, ffn))]


def block_bf16(device="cpu", seed=2, scale=1, first_index=0, prefix=""):
    """BF16 block: matrices N(0, sigma), sigma ~ U[0.008, 0.03] per matrix;
    RMSNorm vectors N(1, 0.05).  scale > 1 divides every dimension (tests)."""
    out = []
    for j, (name, shape) in enumerate(block_shapes(4096 // scale, 1024 // scale, 14336 // scale)):
        i = first_index + j
        n = 1
        for d in shape:
            n *= d
        if name.endswith("norm"):
            t = gaussian(n, 1.0, 0.05, torch.bfloat16, device, seed, i)
        else:
            t = gaussian(n, 0.0, uniform_sigma(0.008, 0.03, seed, i), torch.bfloat16, device, seed, i)
        out.append((prefix + name, t.view(shape)))
    return out


def other_block_bf16(device="cpu", seed=7, scale=1, first_index=0, prefix=""):
    """Another architecture's BF16 block (3B-shaped: hidden 3072, kv 1024, ffn
    8192): matrices N(0, sigma), sigma ~ U[0.01, 0.04] per matrix; RMSNorm
    vectors N(1, 0.05).  scale > 1 divides every dimension (tests)."""
    out = []
    for j, (name, shape) in enumerate(block_shapes(3072 // scale, 1024 // scale, 8192 // scale)):
        i = first_index + j
        n = 1
        for d in shape:
            n *= d
        if name.endswith("norm"):
            t = gaussian(n, 1.0, 0.05, torch.bfloat16, device, seed, i)
        else:
            t = gaussian(n, 0.0, uniform_sigma(0.01, 0.04, seed, i), torch.bfloat16, device, seed, i)
        out.append((prefix + name, t.view(shape)))
    return out


def fp32_pair(n=1 << 27, device="cpu", seed=3):
    """FP32 N(0, 0.02): a regular copy and a clean copy (low 16 fraction bits zero)."""
    reg = gaussian(n, 0.0, 0.02, torch.float32, device, seed, 0)
    clean = (reg.view(torch.int32) & -65536).view(torch.float32)
    return [("regular", reg), ("clean", clean)]


def fp8_blockscaled(n=1 << 30, block=128, device="cpu", seed=4):
    """FP8 E4M3: N(0,1) scaled per 128-element block to max |z| = 448."""
    g = _gen(device, seed, 0)
    out = torch.empty(n, dtype=torch.float8_e4m3fn, device=device)
    step = (GEN_BLOCK // block) * block
    for s in range(0, n, step):
        m = min(step, n - s)
        z = torch.randn(m, dtype=torch.float32, device=device, generator=g)
        nb = (m + block - 1) // block
        zp = torch.zeros(nb * block, dtype=torch.float32, device=device)
        zp[:m] = z
        zb = zp.view(nb, block)
        amax = zb.abs().amax(dim=1, keepdim=True).clamp_min(1e-30)
        y = (zb * (448.0 / amax)).clamp(-448.0, 448.0).reshape(-1)[:m]
        out[s:s + m] = y.to(torch.float8_e4m3fn)
    return [("w_fp8", out)]


# E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); the midpoints
# between neighbours decide the rounding
_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def fp4_blockscaled(n_bytes=1 << 29, block=32, device="cpu", seed=8):
    """FP4 E2M1 pairs (uint8, two values per byte, the first in the low
    nibble): N(0,1) scaled per 32-value block to max |z| = 6, rounded to the
    nearest E2M1 value, ties to the even code."""
    g = _gen(device, seed, 0)
    n = 2 * n_bytes
    out = torch.empty(n_bytes, dtype=torch.uint8, device=device)
    mids = torch.tensor(_E2M1_MIDS, dtype=torch.float64, device=device)
    step = (GEN_BLOCK // (2 * block)) * 2 * block
    for s in range(0, n, step):
        m = min(step, n - s)
        z = torch.randn(m, dtype=torch.float64, device=device, generator=g)
        nb = (m + block - 1) // block
        zp = torch.zeros(nb * block, dtype=torch.float64, device=device)
        zp[:m] = z
        zb = zp.view(nb, block)
        amax = zb.abs().amax(dim=1, keepdim=True).clamp_min(1e-300)
        y = (zb * (6.0 / amax)).reshape(-1)[:m]
        a = y.abs()
        code = torch.bucketize(a, mids)               # mids below a, a tie counted as below
        tie = (code < 7) & (a == mids[code.clamp(max=6)])
        code = code + (tie & (code % 2 == 1)).to(code.dtype)   # a tie goes to the even code
        nib = (code + 8 * (y < 0).to(code.dtype)).to(torch.uint8)
        pair = nib.view(-1, 2)
        out[s // 2:(s + m) // 2] = pair[:, 0] | (pair[:, 1] << 4)
    return [("w_fp4", out)]


def model_bf16(device="cpu", seed=5, n_layers=32, scale=1, with_kv=True, kv_tokens=32768):
    """8B-shaped BF16 model: n_layers blocks + embedding 128256 x 4096 N(0, 0.02)
    + a KV cache [layers, 2, 8 heads, tokens, 128] from N(0, 1)."""
    out = []
    hidden = 4096 // scale
    vocab = 128256 // scale
    out.append(("embed", gaussian(vocab * hidden, 0.0, 0.02, torch.bfloat16, device, seed, 0)
                .view(vocab, hidden)))
    for layer in range(n_layers):
        out += block_bf16(device, seed, scale, first_index=1 + 9 * layer, prefix=f"l{layer}.")
    if with_kv:
        shape = (n_layers, 2, 8, kv_tokens // scale, 128 // scale if scale > 1 else 128)
        n = 1
        for d in shape:
            n *= d
        out.append(("kv", gaussian(n, 0.0, 1.0, torch.bfloat16, device, seed, 999).view(shape)))
    return out


def perturb_bf16(t: torch.Tensor, seed: int, i: int, std=1e-4) -> torch.Tensor:
    """bf16(fp32(w) + N(0, std)) with float64 draws."""
    g = _gen(t.device, seed, 50000 + i)
    flat = t.reshape(-1)
    out = torch.empty_like(flat)
    for s in range(0, flat.numel(), GEN_BLOCK):
        m = min(GEN_BLOCK, flat.numel() - s)
        z = torch.randn(m, dtype=torch.float64, device=t.device, generator=g)
        out[s:s + m] = (flat[s:s + m].to(torch.float32) + (z * std).to(torch.float32)).to(torch.bfloat16)
    return out.view(t.shape)


def perturbed_model(tensors, seed=5):
    """Perturbs every weight; the KV cache is copied unchanged."""
    out = []
    for i, (name, t) in enumerate(tensors):
        out.append((name, t.clone() if name == "kv" else perturb_bf16(t, seed, i)))
    return out
