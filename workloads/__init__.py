"""Seeded synthetic inputs for the verification path.

This module only *draws inputs*: logit tensors of the draft / intermediate /
final exits, drafted tokens, per-sequence temperatures and paged-KV block
tables.  It holds none of the verification arithmetic (no acceptance test, no
residual, no inverse-CDF draw, no rollback).  Tests and the benchmark call it;
the CPU oracle (``oracle/``) and the HIP binding import nothing from it.

Shapes and value laws
---------------------
The pages evaluate on public chat / summarisation / code / math datasets with
Llama, Qwen and OPT models; none of that is available here, so logits are drawn
from seeded laws with the shapes of those workloads instead:

* base logits D at k+1 positions, i.i.d. N(0, std^2) (or scale * Student-t(3));
* a verifier exit correlated with the exit below it:
  target = alpha * below + sqrt(1 - alpha^2) * fresh noise of the same law;
* the draft tensor is D at positions 0..k-1;
* drafted tokens are sampled from the draft rows at the sequence temperature
  (Gumbel-max on the stored logits; argmax at temperature 0);
* bf16 tensors are the float32 draws rounded to nearest-even by torch.

Named workloads (``make(name, trial, device)``):

===========  =====================================================================
tiny          B=1, k=4, V=1024, fp32, std 2, alpha 0.8, temperature 1
batched       B=64, k=4, V=32000, bf16, std 3, alpha_b ~ U[0.5, 0.95], temperature 1
hier          B=256, k=8, V=128256, bf16 L_d/L_i/L_f, std 3, alpha 0.85 (L_i vs
              L_d) and 0.8 (L_f vs L_i), temperature 1, window 4; block tables
              of 16-slot blocks, context ~ U{512..4096}, length = context + k
mixed_temp    B=32, k=5, V=151936, fp32, 4 * Student-t(3), alpha_b ~ U[0.3, 0.99],
              temperature_b uniform over {0, 0.7, 1.0}
lmhead        B=128, k=4, d=4096, V=128256: bf16 hidden states of the draft and final
              exits at k+1 positions, i.i.d. N(0, 1); a shared bf16 LM head W [V, d]
              (one d-vector per vocabulary entry), i.i.d. N(0, 0.02^2); temperature 1;
              drafts sampled from the draft exit's head logits at positions 0..k-1
===========  =====================================================================
"""

import math

import torch

WORKLOADS = {
    "tiny": dict(kind="single", B=1, k=4, V=1024, dtype="f32", law="normal", scale=2.0,
                 alpha=(0.8, 0.8), temps=(1.0,)),
    "batched": dict(kind="single", B=64, k=4, V=32000, dtype="bf16", law="normal", scale=3.0,
                    alpha=(0.5, 0.95), temps=(1.0,)),
    "hier": dict(kind="hier", B=256, k=8, V=128256, dtype="bf16", law="normal", scale=3.0,
                 alpha_i=0.85, alpha_f=0.8, temps=(1.0,), window=4,
                 block_size=16, ctx=(512, 4096)),
    "mixed_temp": dict(kind="single", B=32, k=5, V=151936, dtype="f32", law="t3", scale=4.0,
                       alpha=(0.3, 0.99), temps=(0.0, 0.7, 1.0)),
    "lmhead": dict(kind="lmhead", B=128, k=4, V=128256, d=4096, w_std=0.02, temps=(1.0,)),
}

_IDS = {"tiny": 1, "batched": 2, "hier": 3, "mixed_temp": 4, "lmhead": 5}


def _gen(device, *seed_parts):
    g = torch.Generator(device=device)
    s = 0
    for p in seed_parts:
        s = (s * 1000003 + int(p)) & 0x7FFFFFFFFFFFFFFF
    g.manual_seed(s)
    return g


def _noise(shape, law, scale, g, device):
    if law == "normal":
        return torch.randn(shape, generator=g, device=device) * scale
    if law == "t3":
        z = torch.randn(shape, generator=g, device=device)
        chi2 = torch.zeros(shape, device=device)
        for _ in range(3):
            chi2 += torch.randn(shape, generator=g, device=device) ** 2
        return scale * z / torch.sqrt(chi2 / 3.0)
    raise ValueError(law)


def _store(x, dtype):
    return x.to(torch.bfloat16) if dtype == "bf16" else x.to(torch.float32).contiguous()


def _mix(alpha, below, law, scale, g, device):
    """alpha * below + sqrt(1 - alpha^2) * noise; alpha is a scalar or a [B] tensor."""
    noise = _noise(below.shape, law, scale, g, device)
    if not torch.is_tensor(alpha):
        return alpha * below + math.sqrt(max(0.0, 1.0 - alpha * alpha)) * noise
    a = alpha.view(-1, 1, 1)
    return a * below + torch.sqrt(torch.clamp(1.0 - a * a, min=0.0)) * noise


def _temperatures(B, temps, g, device):
    if len(temps) == 1:
        return torch.full((B,), float(temps[0]), dtype=torch.float32, device=device)
    idx = torch.randint(0, len(temps), (B,), generator=g, device=device)
    return torch.tensor(temps, dtype=torch.float32, device=device)[idx]


def sample_drafts(draft_logits, temperature, g):
    """Drafted tokens from the stored draft logits [B, k, V]: Gumbel-max at
    temperature > 0, argmax (first maximum) at temperature 0."""
    B, k, V = draft_logits.shape
    dev = draft_logits.device
    out = torch.empty((B, k), dtype=torch.int32, device=dev)
    for b in range(B):
        l = draft_logits[b].float()
        tau = float(temperature[b])
        if tau == 0.0:
            out[b] = torch.argmax(l, dim=-1).to(torch.int32)
        else:
            u = torch.rand(l.shape, generator=g, device=dev).clamp_(min=1e-12, max=1.0 - 1e-7)
            gumbel = -torch.log(-torch.log(u))
            out[b] = torch.argmax(l / tau + gumbel, dim=-1).to(torch.int32)
    return out


def block_tables(B, lengths, block_size, max_blocks, g, device="cpu"):
    """Block tables [B, max_blocks] int32 (-1 = empty) holding physical ids
    drawn without replacement from a shuffled pool, enough for each length."""
    need = [(int(L) + block_size - 1) // block_size for L in lengths.tolist()]
    pool = torch.randperm(B * max_blocks, generator=g, device=device).to(torch.int32)
    table = torch.full((B, max_blocks), -1, dtype=torch.int32, device=device)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = pool[pos:pos + n]
        pos += n
    return table


def make_single(B, k, V, dtype="bf16", law="normal", scale=3.0, alpha=(0.5, 0.95),
                temps=(1.0,), seed=(0,), device="cpu"):
    """Single-stage inputs: draft [B,k,V], target [B,k+1,V], tokens, temperatures."""
    g = _gen(device, *seed)
    D = _noise((B, k + 1, V), law, scale, g, device)
    a = torch.empty(B, device=device).uniform_(alpha[0], alpha[1], generator=g)
    T = _mix(a, D, law, scale, g, device)
    temperature = _temperatures(B, temps, g, device)
    draft = _store(D[:, :k].contiguous(), dtype)
    target = _store(T, dtype)
    del D, T
    tokens = sample_drafts(draft, temperature.cpu(), g)
    return dict(kind="single", B=B, k=k, V=V, dtype=dtype, draft_logits=draft,
                target_logits=target, draft_tokens=tokens, temperature=temperature)


def make_hier(B, k, V, dtype="bf16", law="normal", scale=3.0, alpha_i=0.85, alpha_f=0.8,
              temps=(1.0,), window=4, block_size=16, ctx=(512, 4096), seed=(0,),
              device="cpu"):
    """Hierarchical inputs: L_d [B,k,V], L_i and L_f [B,k+1,V], tokens,
    temperatures, plus a paged-KV state (block_table, seq_lens)."""
    g = _gen(device, *seed)
    D = _noise((B, k + 1, V), law, scale, g, device)
    Li = _mix(alpha_i, D, law, scale, g, device)
    ld = _store(D[:, :k].contiguous(), dtype)
    del D
    Lf = _mix(alpha_f, Li, law, scale, g, device)
    li = _store(Li, dtype)
    del Li
    lf = _store(Lf, dtype)
    del Lf
    temperature = _temperatures(B, temps, g, device)
    tokens = sample_drafts(ld, temperature.cpu(), g)
    gc = _gen("cpu", *seed, 77)
    context = torch.randint(ctx[0], ctx[1] + 1, (B,), generator=gc)
    seq_lens = (context + k).to(torch.int32)
    max_blocks = (ctx[1] + k + block_size - 1) // block_size
    table = block_tables(B, seq_lens, block_size, max_blocks, gc)
    return dict(kind="hier", B=B, k=k, V=V, dtype=dtype, ld_logits=ld, li_logits=li,
                lf_logits=lf, draft_tokens=tokens, temperature=temperature, window=window,
                block_size=block_size, block_table=table.to(device),
                seq_lens=seq_lens.to(device), max_blocks=max_blocks)


def make_lmhead(B, k, V, d, w_std=0.02, temps=(1.0,), seed=(0,), device="cpu"):
    """LM-head inputs: hidden states h_draft [B, k, d] (the draft exit at the k
    drafted positions), h_target [B, k+1, d], head w_vocab [V, d] (bf16), drafted
    tokens sampled from the draft exit's head logits (float32, test side), and
    temperatures."""
    g = _gen(device, *seed)
    hd = torch.randn((B, k + 1, d), generator=g, device=device).to(torch.bfloat16)
    ht = torch.randn((B, k + 1, d), generator=g, device=device).to(torch.bfloat16)
    w = torch.empty((V, d), dtype=torch.bfloat16, device=device)
    for v0 in range(0, V, 16384):                     # bounded float32 temporaries
        v1 = min(V, v0 + 16384)
        w[v0:v1] = (torch.randn((v1 - v0, d), generator=g, device=device) * w_std).to(torch.bfloat16)
    temperature = _temperatures(B, temps, g, device)
    h_draft = hd[:, :k].contiguous()
    tokens = torch.empty((B, k), dtype=torch.int32, device=device)
    wf = w.float()
    for b0 in range(0, B, 16):
        b1 = min(B, b0 + 16)
        logits = (h_draft[b0:b1].float().reshape(-1, d) @ wf.T).reshape(b1 - b0, k, V)
        tokens[b0:b1] = sample_drafts(logits, temperature[b0:b1].cpu(), g)
    del wf
    return dict(kind="lmhead", B=B, k=k, V=V, d=d, dtype="bf16", h_draft=h_draft,
                h_target=ht, w_vocab=w, draft_tokens=tokens, temperature=temperature)


def make(name, trial=0, device="cpu"):
    """A named workload (see the module docstring) for a given trial index."""
    cfg = dict(WORKLOADS[name])
    kind = cfg.pop("kind")
    seed = (_IDS[name], trial)
    if kind == "single":
        return make_single(seed=seed, device=device, **cfg)
    if kind == "lmhead":
        return make_lmhead(seed=seed, device=device, **cfg)
    return make_hier(seed=seed, device=device, **cfg)


def to_numpy_raw(t):
    """Tensor -> NumPy raw logits as the oracle takes them: uint16 bf16 bits or
    float32 values."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
