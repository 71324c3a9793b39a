"""Workload shapes of the int4 GPTQ linear layer and the dense training products.

The int4 shapes are the (k, n) pairs the GPTQModel NF12 pull request measures
its fused small-M kernel on (its same-process A/B table and its table against
dense BF16), with the token counts m at which it switches between kernels.  The
dense shapes are the per-layer training products of the BC-250 tuned-GEMM post
("Tuning the kernels": every layer at 1,024, 2,048 and 4,096 tokens and the
rank-16 LoRA matrices) for a model with hidden size 2048 and FFN size 5632.

The batched attention products (the same post tunes "the batched products
inside attention" and validates batched attention shapes) are taken at the same
token counts for one sequence whose hidden size 2048 is split into 32 heads of
64 (the pages give no head layout; this split is a reading): per head the
scores S = Q K^T, the output O = P V, and the gradients dP = dO V^T,
dV = P^T dO, dQ = dS K and dK = dS^T Q.

Seeds: case i of config c uses seed (1000 + c) * 65536 + i (attention: c = 5).
"""
from __future__ import annotations

INT4_CONFIGS = {
    # GEMV: one token, a small projection.
    0: {"name": "int4 GEMV k=896 n=4864", "shapes": [(896, 4864)], "m": [1]},
    # small-M: the fused-kernel regime.
    1: {"name": "int4 small-M", "shapes": [(4096, 4096), (2048, 8192)], "m": [1, 8, 15]},
    # prefill through MFMA.
    2: {"name": "int4 prefill", "shapes": [(25600, 5120), (5120, 25600)], "m": [16, 512, 2048]},
    # large weights (LLC pressure).
    4: {"name": "int4 large weights", "shapes": [(4096, 28672), (4096, 14336), (8192, 8192)],
        "m": [1, 8, 16]},
}

DENSE_CONFIGS = {
    3: {"name": "dense training trio", "tokens": [1024, 2048, 4096],
        # weight matrices W[n][k] of the FFN: up/gate [5632][2048], down [2048][5632]
        "weights": [(5632, 2048), (2048, 5632)], "dtypes": ["bf16", "fp16"], "lora_rank": 16},
}


ATTENTION_CONFIG = {"name": "batched attention products", "tokens": [1024, 2048, 4096], "heads": 32,
                    "head_dim": 64, "dtypes": ["bf16", "fp16"], "std": 1.0}


def seed_for(config: int, case: int) -> int:
    return (1000 + config) * 65536 + case


def int4_cases(config: int):
    """List of (case_index, m, k, n, seed) of an int4 config, shape-major."""
    c = INT4_CONFIGS[config]
    out = []
    i = 0
    for (k, n) in c["shapes"]:
        for m in c["m"]:
            out.append((i, m, k, n, seed_for(config, i)))
            i += 1
    return out


def dense_cases(config: int = 3, with_lora: bool = True):
    """List of dict(layout, dtype, M, N, K, seed, role) for the training trio.

    For a weight W[n][k] and t tokens:
      forward  NT  M=t  N=n  K=k
      dgrad    NN  M=t  N=k  K=n
      wgrad    TN  M=n  N=k  K=t
    and the rank-r LoRA products with adapters A_l[r][k], B_l[n][r]:
      U = X A_l^T (NT t,r,k);  Y += U B_l^T (NT t,n,r)
      dU = dY B_l (NN t,r,n);  dX += dU A_l (NN t,k,r)
      dB_l = dY^T U (TN n,r,t);  dA_l = dU^T X (TN r,k,t)
    """
    c = DENSE_CONFIGS[config]
    r = c["lora_rank"]
    out = []
    i = 0
    for dtype in c["dtypes"]:
        for t in c["tokens"]:
            for (n, k) in c["weights"]:
                prods = [("forward", "NT", t, n, k), ("dgrad", "NN", t, k, n),
                         ("wgrad", "TN", n, k, t)]
                if with_lora:
                    prods += [("lora_u", "NT", t, r, k), ("lora_y", "NT", t, n, r),
                              ("lora_du", "NN", t, r, n), ("lora_dx", "NN", t, k, r),
                              ("lora_db", "TN", n, r, t), ("lora_da", "TN", r, k, t)]
                for role, layout, M, N, K in prods:
                    out.append({"role": role, "layout": layout, "dtype": dtype, "M": M,
                                "N": N, "K": K, "t": t, "w": (n, k),
                                "seed": seed_for(config, i)})
                    i += 1
    return out


def attention_cases():
    """List of dict(role, layout, dtype, batch, M, N, K, seed, t) of the attention products.

    For t tokens, h heads of width d (operands [h][t][d] or [h][t][t]):
      scores  NT  M=t N=t K=d     (Q K^T)
      pv      NN  M=t N=d K=t     (P V)
      dp      NT  M=t N=t K=d     (dO V^T)
      dv      TN  M=t N=d K=t     (P^T dO)
      dq      NN  M=t N=d K=t     (dS K)
      dk      TN  M=t N=d K=t     (dS^T Q)
    """
    c = ATTENTION_CONFIG
    h, d = c["heads"], c["head_dim"]
    out = []
    i = 0
    for dtype in c["dtypes"]:
        for t in c["tokens"]:
            for role, layout, M, N, K in (("scores", "NT", t, t, d), ("pv", "NN", t, d, t),
                                          ("dp", "NT", t, t, d), ("dv", "TN", t, d, t),
                                          ("dq", "NN", t, d, t), ("dk", "TN", t, d, t)):
                out.append({"role": role, "layout": layout, "dtype": dtype, "batch": h, "M": M,
                            "N": N, "K": K, "t": t, "seed": seed_for(5, i)})
                i += 1
    return out
