"""An independent fp64 decoder written with torch library routines.

Used only to pin the oracle: it shares nothing with oracle.cpp.  It computes a
full causal forward over a whole prompt (no KV cache) with
torch.nn.functional's rms_norm / linear / scaled_dot_product_attention / silu,
RoPE as a complex rotation (torch.polar), and the routed MLP via torch.topk on
softmax probabilities.  Keys and values are rounded to bf16 before attention,
as the decoder's bf16 cache stores them.
"""

import numpy as np
import torch
import torch.nn.functional as F


def _w(ws, name):
    a = ws[name]
    t = torch.from_numpy((a.astype(np.uint32) << 16).view(np.float32)).to(torch.float64)
    return t


def _rope_complex(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    # x [..., T, D]; pair i is (x_i, x_{i+D/2}) read as the complex number x_i + j x_{i+D/2}
    D = x.shape[-1]
    h = D // 2
    freqs = theta ** (-2.0 * torch.arange(h, dtype=torch.float64) / D)
    ang = pos.to(torch.float64)[:, None] * freqs[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)  # e^{j ang}
    z = torch.complex(x[..., :h], x[..., h:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def _round_bf16(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def forward_last_logits(shape, ws, tokens, forced_last=None, router_out=None) -> np.ndarray:
    """Logits (float64, [V]) at the last position of `tokens` (positions 0..n-1).

    Routed models: ``forced_last[l]`` (optional) is the expert choice of layer l
    at the last position, weighted by its softmax probabilities renormalised
    over the choice; earlier positions always take the top-k.  If given,
    ``router_out`` (a list) receives the router logits [E] of the last position
    per layer."""
    s = shape
    H, D, Hq, Hkv = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads
    G = Hq // Hkv
    n = len(tokens)
    pos = torch.arange(n)
    emb = _w(ws, "embed").reshape(s.vocab, H)
    x = emb[torch.as_tensor(np.asarray(tokens, dtype=np.int64))]  # [n, H]
    eps = s.rms_eps
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    for l in range(s.n_layers):
        p = f"layers.{l}."
        h = F.rms_norm(x, (H,), weight=_w(ws, p + "in_norm"), eps=eps)
        q = F.linear(h, _w(ws, p + "wq").reshape(Hq * D, H)).reshape(n, Hq, D).transpose(0, 1)
        k = F.linear(h, _w(ws, p + "wk").reshape(Hkv * D, H)).reshape(n, Hkv, D).transpose(0, 1)
        v = F.linear(h, _w(ws, p + "wv").reshape(Hkv * D, H)).reshape(n, Hkv, D).transpose(0, 1)
        q = F.rms_norm(q, (D,), weight=_w(ws, p + "q_norm"), eps=eps)
        k = F.rms_norm(k, (D,), weight=_w(ws, p + "k_norm"), eps=eps)
        q = _rope_complex(q, pos, s.rope_theta)
        k = _round_bf16(_rope_complex(k, pos, s.rope_theta))
        v = _round_bf16(v)
        k = k.repeat_interleave(G, dim=0).contiguous()
        v = v.repeat_interleave(G, dim=0).contiguous()
        o = F.scaled_dot_product_attention(q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0),
                                           attn_mask=mask).squeeze(0)  # [Hq, n, D]
        o = o.transpose(0, 1).reshape(n, Hq * D)
        x = x + F.linear(o, _w(ws, p + "wo").reshape(H, Hq * D))
        h2 = F.rms_norm(x, (H,), weight=_w(ws, p + "post_norm"), eps=eps)
        if s.n_experts == 0:
            I = s.intermediate
            a = F.silu(F.linear(h2, _w(ws, p + "w_gate").reshape(I, H))) * F.linear(h2, _w(ws, p + "w_up").reshape(I, H))
            x = x + F.linear(a, _w(ws, p + "w_down").reshape(H, I))
        else:
            Ie, E, K = s.expert_intermediate, s.n_experts, s.top_k
            rl = F.linear(h2, _w(ws, p + "router").reshape(E, H))
            if router_out is not None:
                router_out.append(rl[-1].numpy().copy())
            probs = torch.softmax(rl, dim=-1)
            top_p, top_e = torch.topk(probs, K, dim=-1)
            if forced_last is not None:
                top_e[-1] = torch.as_tensor(np.asarray(forced_last[l], dtype=np.int64))
                top_p[-1] = probs[-1, top_e[-1]]
            top_p = top_p / top_p.sum(dim=-1, keepdim=True)
            y = torch.zeros_like(x)
            for t in range(n):
                for j in range(K):
                    e = int(top_e[t, j])
                    q_ = p + f"experts.{e}."
                    a = F.silu(F.linear(h2[t], _w(ws, q_ + "w_gate").reshape(Ie, H))) * \
                        F.linear(h2[t], _w(ws, q_ + "w_up").reshape(Ie, H))
                    y[t] += top_p[t, j] * F.linear(a, _w(ws, q_ + "w_down").reshape(H, Ie))
            x = x + y
    hf = F.rms_norm(x[-1], (H,), weight=_w(ws, "final_norm"), eps=eps)
    W = _w(ws, "embed" if s.tied_embeddings else "lm_head").reshape(s.vocab, H)
    return F.linear(hf, W).numpy()
