"""An independent statement of the encoder built from torch's own layers.

Used only by CPU tests to pin the oracle: torch.nn.functional.conv1d /
gelu / layer_norm and torch.nn.TransformerEncoderLayer (pre-norm, exact
GELU) in float64 compute the same function as the pages describe, through
code that shares nothing with ``oracle/``.
"""
import numpy as np
import torch
import torch.nn.functional as F


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64).copy())


def torch_block(d, n_head, d_ff, eps, p):
    layer = torch.nn.TransformerEncoderLayer(
        d, n_head, dim_feedforward=d_ff, dropout=0.0, activation="gelu",
        layer_norm_eps=eps, batch_first=True, norm_first=True, dtype=torch.float64)
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(torch.cat([_t(p["wq"]), _t(p["wk"]), _t(p["wv"])]))
        # k_proj has no bias: a zero bias in the packed in-projection
        layer.self_attn.in_proj_bias.copy_(torch.cat([_t(p["bq"]), torch.zeros(d, dtype=torch.float64), _t(p["bv"])]))
        layer.self_attn.out_proj.weight.copy_(_t(p["wo"]))
        layer.self_attn.out_proj.bias.copy_(_t(p["bo"]))
        layer.linear1.weight.copy_(_t(p["fc1_w"]))
        layer.linear1.bias.copy_(_t(p["fc1_b"]))
        layer.linear2.weight.copy_(_t(p["fc2_w"]))
        layer.linear2.bias.copy_(_t(p["fc2_b"]))
        layer.norm1.weight.copy_(_t(p["ln1_g"]))
        layer.norm1.bias.copy_(_t(p["ln1_b"]))
        layer.norm2.weight.copy_(_t(p["ln2_g"]))
        layer.norm2.bias.copy_(_t(p["ln2_b"]))
    layer.train(False)
    return layer


def torch_encode(mel, params, n_layer, n_head, eps=1e-5, final_ln=True):
    """mel [T_in, n_mels] -> [T_in // 2, d] float64 numpy."""
    x = _t(mel).T.unsqueeze(0)  # [1, n_mels, T_in]
    d = params["conv1_w"].shape[0]
    with torch.no_grad():
        c1 = F.gelu(F.conv1d(x, _t(params["conv1_w"]), _t(params["conv1_b"]), stride=1, padding=1))
        c2 = F.gelu(F.conv1d(c1, _t(params["conv2_w"]), _t(params["conv2_b"]), stride=2, padding=1))
        h = c2[0].T
        h = h + _t(params["pos"])[:h.shape[0]]  # a shortened window uses the leading rows
        for li in range(n_layer):
            p = {k.split(".", 1)[1]: v for k, v in params.items() if k.startswith(f"l{li}.")}
            d_ff = p["fc1_w"].shape[0]
            h = torch_block(d, n_head, d_ff, eps, p)(h.unsqueeze(0)).squeeze(0)
        if final_ln:
            h = F.layer_norm(h, (d,), _t(params["lnf_g"]), _t(params["lnf_b"]), eps)
    return h.numpy()
