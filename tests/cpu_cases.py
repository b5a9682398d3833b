"""Test-side builders: scatter logical K/V into a paged pool with explicit per-token loops, and
decode storage bits with torch's own dtypes.  Kept apart from the oracle on purpose: the pins
compare the oracle against these independent routes."""

from __future__ import annotations

import numpy as np
import torch

BLOCK = 16
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "fp8_e4m3": torch.float8_e4m3fn}


def torch_decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage bits -> float64 through torch's dtype conversion."""
    a = np.ascontiguousarray(bits)
    if dtype == "fp8_e4m3":
        t = torch.from_numpy(a.view(np.uint8)).view(torch.float8_e4m3fn)
    else:
        t = torch.from_numpy(a.view(np.int16)).view(TORCH_DT[dtype])
    return t.to(torch.float64).numpy()


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    if dtype == "fp8_e4m3":
        return t.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return t.to(TORCH_DT[dtype]).view(torch.int16).numpy().view(np.uint16).copy()


class Case:
    """A paged pool built from logical per-sequence K/V by explicit scatter loops."""

    def __init__(self, rng, lens, Hkv, G, D, kv_dtype="bf16", q_dtype="bf16", pool_blocks=None,
                 tables=None, scale=None):
        self.lens = np.asarray(lens, dtype=np.int32)
        B = len(lens)
        self.B, self.Hkv, self.G, self.D = B, Hkv, G, D
        self.Hq = Hkv * G
        self.kv_dtype, self.q_dtype = kv_dtype, q_dtype
        nblk = [-(-int(L) // BLOCK) for L in lens]
        need = sum(nblk)
        NB = pool_blocks if pool_blocks is not None else 2 * need + 3
        self.NB = NB
        if tables is None:
            perm = rng.permutation(NB)
            tables, c = [], 0
            for n in nblk:
                tables.append(list(perm[c:c + n]))
                c += n
        MB = max(1, max(len(t) for t in tables))
        self.tables = np.zeros((B, MB), dtype=np.int32)
        for b, t in enumerate(tables):
            self.tables[b, :len(t)] = t
        bits_t = np.uint8 if kv_dtype == "fp8_e4m3" else np.uint16
        nan = bits_t(0x7F if kv_dtype == "fp8_e4m3" else (0x7FC0 if kv_dtype == "bf16" else 0x7E00))
        self.k_cache = np.full((NB, Hkv, BLOCK, D), nan, dtype=bits_t)
        self.v_cache = np.full((NB, Hkv, D, BLOCK), nan, dtype=bits_t)
        self.k_scale = self.v_scale = None
        if kv_dtype == "fp8_e4m3":
            self.k_scale = np.full((NB, Hkv), np.nan, dtype=np.float32)
            self.v_scale = np.full((NB, Hkv), np.nan, dtype=np.float32)
        # logical values (float64, exactly the stored values)
        self.q_bits = round_bits(rng.standard_normal((B, self.Hq, D)), q_dtype)
        self.q = torch_decode(self.q_bits, q_dtype)
        self.K, self.V = [], []
        for b in range(B):
            L = int(lens[b])
            Kb = np.zeros((Hkv, L, D))
            Vb = np.zeros((Hkv, L, D))
            kbits = round_bits(rng.standard_normal((Hkv, L, D)) * 4 if kv_dtype == "fp8_e4m3"
                               else rng.standard_normal((Hkv, L, D)), kv_dtype)
            vbits = round_bits(rng.standard_normal((Hkv, L, D)) * 4 if kv_dtype == "fp8_e4m3"
                               else rng.standard_normal((Hkv, L, D)), kv_dtype)
            for j in range(nblk[b]):
                blk = int(self.tables[b, j])
                for h in range(Hkv):
                    ks = vs = 1.0
                    if kv_dtype == "fp8_e4m3":
                        ks = float(np.float32(rng.uniform(0.01, 0.5)))
                        vs = float(np.float32(rng.uniform(0.01, 0.5)))
                        self.k_scale[blk, h] = ks
                        self.v_scale[blk, h] = vs
                    for off in range(BLOCK):
                        t = j * BLOCK + off
                        if t >= L:
                            break
                        self.k_cache[blk, h, off, :] = kbits[h, t]
                        for d in range(D):
                            self.v_cache[blk, h, d, off] = vbits[h, t, d]
                        Kb[h, t] = torch_decode(kbits[h, t], kv_dtype) * ks
                        Vb[h, t] = torch_decode(vbits[h, t], kv_dtype) * vs
            self.K.append(Kb)
            self.V.append(Vb)
        self.scale = np.float32(1.0 / np.sqrt(D)) if scale is None else np.float32(scale)

    def sdpa(self) -> np.ndarray:
        """torch scaled_dot_product_attention on the contiguous logical arrays (float64)."""
        out = np.zeros((self.B, self.Hq, self.D))
        for b in range(self.B):
            L = int(self.lens[b])
            if L == 0:
                continue
            for h in range(self.Hq):
                kvh = h // self.G
                q = torch.from_numpy(self.q[b, h]).view(1, 1, 1, self.D)
                k = torch.from_numpy(self.K[b][kvh]).view(1, 1, L, self.D)
                v = torch.from_numpy(self.V[b][kvh]).view(1, 1, L, self.D)
                o = torch.nn.functional.scaled_dot_product_attention(
                    q, k, v, scale=float(self.scale))
                out[b, h] = o.view(self.D).numpy()
        return out

    def oracle_args(self):
        return dict(q=self.q_bits, k_cache=self.k_cache, v_cache=self.v_cache,
                    block_tables=self.tables, context_lens=self.lens, scale=self.scale,
                    q_dtype=self.q_dtype, kv_dtype=self.kv_dtype,
                    k_scale=self.k_scale, v_scale=self.v_scale)
