"""Seeded generators.  Values are drawn in float64 with torch's generator on
the target device (numpy-free so full-size workloads can be drawn on the GPU),
then rounded once to the storage dtype (round-to-nearest-even for bf16).
Draw order is fixed: [lengths], q, k, v, beta logits, alpha logits, S0."""
import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device, mean=0.0, std=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float64)
    return x * std + mean if (mean != 0.0 or std != 1.0) else x


def _unit(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def _alpha(lead, dk, gate, g, device, mu, sigma=1.0, logits=False, dtype=torch.float32):
    """Forget gates sigmoid(N(mu, sigma)): [*lead, dk] per channel, [*lead]
    per head, None without a gate (nothing drawn).  logits=True stores the
    N(mu, sigma) draws themselves in ``dtype``."""
    if gate == "none":
        return None
    shape = tuple(lead) + ((dk,) if gate == "channel" else ())
    if gate not in ("channel", "head"):
        raise ValueError("unknown gate %r" % (gate,))
    z = _normal(shape, g, device, mu, sigma)
    if logits:
        return z.to(dtype).contiguous()
    return torch.sigmoid(z).to(torch.float32).contiguous()


def draw_chunk(B, T, H, dk, dv, dtype="bf16", alpha_mu=4.0, alpha_sigma=1.0, s0_std=None,
               num_states=None, seed=0, device="cpu", lengths=None, gate="channel",
               raw=False):
    """Draw one chunked-forward input set.

    Returns a dict with q, k [B,T,H,dk] and v [B,T,H,dv] in the storage dtype,
    alpha [B,T,H,dk] (gate "channel"), [B,T,H] ("head") or None ("none") and
    beta [B,T,H] in float32, initial_state [num_states or B, H, dk, dv]
    float32 (or None), on ``device``.  raw=True draws the same values but
    stores what in-kernel preparation takes: q and k not normalised, and
    the logits of alpha (in the storage dtype) and of beta (float32).
    """
    g = _gen(device, seed)
    dt = _DT[dtype]
    prep = (lambda x: x) if raw else _unit
    q = prep(_normal((B, T, H, dk), g, device)).to(dt)
    k = prep(_normal((B, T, H, dk), g, device)).to(dt)
    v = _normal((B, T, H, dv), g, device).to(dt)
    beta = _normal((B, T, H), g, device)
    beta = (beta if raw else torch.sigmoid(beta)).to(torch.float32)
    alpha = _alpha((B, T, H), dk, gate, g, device, alpha_mu, alpha_sigma, logits=raw,
                   dtype=dt)
    ns = B if num_states is None else num_states
    s0 = None
    if s0_std is not None:
        s0 = _normal((ns, H, dk, dv), g, device, 0.0, s0_std).to(torch.float32)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), alpha=alpha,
                beta=beta.contiguous(), initial_state=s0, gate=gate, raw=raw)


def varlen_lengths(num_seqs, lo, hi, seed):
    """Integer lengths uniform on [lo, hi] inclusive, drawn on the CPU."""
    g = _gen("cpu", 1000003 + int(seed))
    return [int(x) for x in torch.randint(lo, hi + 1, (num_seqs,), generator=g)]


def chunk_inputs(cfg, device="cpu", T=None, B=None, H=None, seed=None, gate="channel",
                 raw=False):
    """Inputs of a chunked-forward workload; T/B/H override the sizes for
    reduced versions and ``gate`` the forget gate's granularity (the same
    draws otherwise).  Varlen workloads also get cu_seqlens (host list and an
    int32 tensor on ``device``)."""
    seed = cfg.seed if seed is None else seed
    H = cfg.H if H is None else H
    if cfg.num_seqs:
        lens = varlen_lengths(cfg.num_seqs, cfg.len_range[0], cfg.len_range[1], seed)
        if T is not None:  # reduced: scale every length down, keep the mix
            total = sum(lens)
            lens = [max(1, (l * T) // total) for l in lens]
        cu = [0]
        for l in lens:
            cu.append(cu[-1] + l)
        d = draw_chunk(1, cu[-1], H, cfg.dk, cfg.dv, cfg.dtype, cfg.alpha_mu, 1.0, cfg.s0_std,
                       num_states=len(lens), seed=seed, device=device, gate=gate, raw=raw)
        d["cu_seqlens_host"] = cu
        d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=device)
        return d
    d = draw_chunk(cfg.B if B is None else B, cfg.T if T is None else T, H, cfg.dk, cfg.dv,
                   cfg.dtype, cfg.alpha_mu, 1.0, cfg.s0_std, seed=seed, device=device, gate=gate,
                   raw=raw)
    d["cu_seqlens_host"] = None
    d["cu_seqlens"] = None
    return d


def decode_inputs(cfg, device="cpu", N=None, H=None, steps=None, seed=None, gate="channel",
                  raw=False):
    """Decode workload: initial state [N,H,dk,dv] float32 and per-step inputs
    stacked on a leading step axis: q, k [S,N,H,dk], v [S,N,H,dv] (storage
    dtype), alpha [S,N,H,dk] (gate "channel"), [S,N,H] ("head") or None
    ("none"), beta [S,N,H] float32."""
    seed = cfg.seed if seed is None else seed
    N = cfg.B if N is None else N
    H = cfg.H if H is None else H
    steps = cfg.steps if steps is None else steps
    g = _gen(device, seed)
    dt = _DT[cfg.dtype]
    state = _normal((N, H, cfg.dk, cfg.dv), g, device, 0.0, cfg.s0_std).to(torch.float32)
    prep = (lambda x: x) if raw else _unit
    q = prep(_normal((steps, N, H, cfg.dk), g, device)).to(dt)
    k = prep(_normal((steps, N, H, cfg.dk), g, device)).to(dt)
    v = _normal((steps, N, H, cfg.dv), g, device).to(dt)
    beta = _normal((steps, N, H), g, device)
    beta = (beta if raw else torch.sigmoid(beta)).to(torch.float32)
    alpha = _alpha((steps, N, H), cfg.dk, gate, g, device, cfg.alpha_mu, logits=raw, dtype=dt)
    return dict(state=state.contiguous(), q=q.contiguous(), k=k.contiguous(), v=v.contiguous(),
                alpha=alpha, beta=beta.contiguous(), gate=gate, raw=raw)


def draw_gdn2(B, T, H, dk, dv, dtype="bf16", alpha_mu=4.0, s0_std=None, num_states=None, seed=0,
              device="cpu", forget=True):
    """Gated DeltaNet-2 inputs: q, k (L2-normalised), v as for draw_chunk; alpha =
    sigmoid(N(alpha_mu, 1)) per key channel (None with forget=False); erase and
    write gates sigmoid(N(0, 1)) per key channel (drawn like beta, one per
    channel); all gates float32 [B, T, H, dk].  Draw order: q, k, v, erase,
    write, alpha, S0."""
    g = _gen(device, seed)
    dt = _DT[dtype]
    q = _unit(_normal((B, T, H, dk), g, device)).to(dt)
    k = _unit(_normal((B, T, H, dk), g, device)).to(dt)
    v = _normal((B, T, H, dv), g, device).to(dt)
    erase = torch.sigmoid(_normal((B, T, H, dk), g, device)).to(torch.float32)
    write = torch.sigmoid(_normal((B, T, H, dk), g, device)).to(torch.float32)
    alpha = (torch.sigmoid(_normal((B, T, H, dk), g, device, alpha_mu)).to(torch.float32)
             if forget else None)
    ns = B if num_states is None else num_states
    s0 = None
    if s0_std is not None:
        s0 = _normal((ns, H, dk, dv), g, device, 0.0, s0_std).to(torch.float32)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), alpha=alpha,
                erase=erase.contiguous(), write=write.contiguous(), initial_state=s0)
