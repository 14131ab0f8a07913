"""Second formulation of the draft step from torch library routines (float64,
CPU).  Used only as a pin for the oracle: torch's rms_norm, complex-number
rotation for RoPE, scaled_dot_product_attention (no mask, GQA by head
repetition), silu and linear.  Shares nothing with oracle/."""
import torch
import torch.nn.functional as Fn

T = torch.float64


def t(a):
    return torch.as_tensor(a).to(T)


def rms(x, g, eps):
    return Fn.rms_norm(x, (x.shape[-1],), weight=t(g), eps=eps)


def rope_complex(x, pos, base):
    """x [..., T, hd]: channel i pairs with i + hd/2 as a complex number
    x_i + 1j * x_{i+hd/2}, multiplied by exp(1j * pos * base**(-2i/hd))."""
    hd = x.shape[-1]
    half = hd // 2
    z = torch.complex(x[..., :half], x[..., half:])
    inv = torch.tensor(base, dtype=T) ** (-(torch.arange(half, dtype=T) * 2) / hd)
    ang = t(pos)[:, None] * inv[None, :]
    r = z * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([r.real, r.imag], dim=-1)


def sdpa(q, K, V, G):
    """q [Hq, B, hd], K/V [Hkv, T, hd] -> [B, Hq*hd] via torch SDPA, no mask."""
    Kx = K.repeat_interleave(G, dim=0)
    Vx = V.repeat_interleave(G, dim=0)
    o = Fn.scaled_dot_product_attention(q[None], Kx[None], Vx[None], attn_mask=None,
                                        is_causal=False)[0]
    return o.transpose(0, 1).reshape(q.shape[1], -1)


def fuse(w, d, hidden):
    z = sum(Fn.linear(t(h), t(w["w_c"])[:, l * d.Dt:(l + 1) * d.Dt]) for l, h in enumerate(hidden))
    return rms(z, w["g_c"], d.rms_eps)


def forward(w, d, hidden_ctx, anchor):
    """Fuse `hidden_ctx` (positions 0..ctx-1), then draft one block; returns
    logits [B-1, V]."""
    B = d.B
    ctx = hidden_ctx[0].shape[0]
    Kc, Vc = [], []
    if ctx:
        Hc = fuse(w, d, hidden_ctx)
    for lw in w["layers"]:
        if ctx:
            k = Fn.linear(Hc, t(lw["w_kc"])).reshape(ctx, d.Hkv, d.hd).transpose(0, 1)
            v = Fn.linear(Hc, t(lw["w_vc"])).reshape(ctx, d.Hkv, d.hd).transpose(0, 1)
            if d.use_rope:
                k = rope_complex(k, torch.arange(ctx), d.rope_base)
        else:
            k = torch.zeros(d.Hkv, 0, d.hd, dtype=T)
            v = torch.zeros(d.Hkv, 0, d.hd, dtype=T)
        Kc.append(k)
        Vc.append(v)
    x = torch.stack([t(w["embed"][anchor])] + [t(w["e_mask"])] * (B - 1))
    pos = torch.arange(ctx, ctx + B)
    for l, lw in enumerate(w["layers"]):
        u = rms(x, lw["g_attn"], d.rms_eps)
        q = Fn.linear(u, t(lw["w_q"])).reshape(B, d.Hq, d.hd).transpose(0, 1)
        kb = Fn.linear(u, t(lw["w_kb"])).reshape(B, d.Hkv, d.hd).transpose(0, 1)
        vb = Fn.linear(u, t(lw["w_vb"])).reshape(B, d.Hkv, d.hd).transpose(0, 1)
        if d.use_rope:
            q = rope_complex(q, pos, d.rope_base)
            kb = rope_complex(kb, pos, d.rope_base)
        o = sdpa(q, torch.cat([Kc[l], kb], 1), torch.cat([Vc[l], vb], 1), d.G)
        x = x + Fn.linear(o, t(lw["w_o"]))
        u = rms(x, lw["g_ffn"], d.rms_eps)
        x = x + Fn.linear(Fn.silu(Fn.linear(u, t(lw["w_gate"]))) * Fn.linear(u, t(lw["w_up"])),
                          t(lw["w_down"]))
    h = rms(x[1:], w["g_final"], d.rms_eps)
    return Fn.linear(h, t(w["w_lm"])).numpy()
