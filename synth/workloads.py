"""Seeded synthetic workloads with the shapes of the CoMERA pages' models.

The pages train a six-encoder transformer (sequence length 128, every linear
layer tensorised, ranks starting at 30), a DLRM with tensorised embedding
tables, and a CodeBERT-large-shaped model (CoMERA project page, "Results").
Their datasets are not available, so every input here is random with the
shapes, value distributions and rank-mask structure of those layers.

Seeds: numpy PCG64 seeded with SeedSequence([config, layer, tensor_id,
BASE_SEED]), so any layer of any configuration can be regenerated on its own.

Readings of the workload descriptions:

* the link diagonals draw U(0.5, 1.5) and then exactly floor(p * r) entries
  per link, picked by a seeded permutation, are set to 0;
* core entries are N(0, sigma^2) with one sigma per layer, chosen so that the
  reconstructed W has entry variance 1 / N_in given the drawn D:
  E[W_ij^2] = sigma^(2d) * prod_k sum_a D_k[a]^2;
* each layer gets its own independent x and dY, N(0, 1);
* bf16 values are the fp32 draws rounded to nearest-even; fp8 values the
  fp32 draws rounded to the nearest OCP e4m3 value (ties to the even code);
  cores and D stay fp32 (master weights), only activations are stored in
  bf16 or fp8;
* TTM ids follow a finite Zipf law P(k) ~ (k+1)^-s over the vocabulary,
  sampled by inverse CDF from seeded uniforms.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BASE_SEED = 20241202

# tensor ids inside one layer's seed sequence
_T_DVAL, _T_DZERO, _T_CORES, _T_X, _T_DY, _T_IDS = 0, 1, 2, 3, 4, 5


def _rng(config: int, layer: int, tensor: int, base: int = BASE_SEED) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config, layer, tensor, base])))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Works in chunks so that large activations need no full-size temporaries.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 20
    for s in range(0, u.size, step):
        c = u[s:s + step]
        bias = np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))
        out[s:s + step] = (c + bias) >> np.uint32(16)
    return out.reshape(np.shape(a))


def _e4m3_table() -> np.ndarray:
    """Values of the 127 non-negative finite OCP e4m3 codes 0x00..0x7E, ascending
    (4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal;
    0x7F is NaN, so 448 is the largest finite value)."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e - 10))


_E4M3 = _e4m3_table()


def fp8_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3 codes (uint8), round to nearest, ties to the even code
    (even mantissa), magnitudes above 448 saturated to 448."""
    x = np.asarray(a, dtype=np.float64)
    ax = np.minimum(np.abs(x), _E4M3[-1])
    hi = np.clip(np.searchsorted(_E4M3, ax), 1, 126)
    lo = hi - 1
    dlo, dhi = ax - _E4M3[lo], _E4M3[hi] - ax
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(ax == _E4M3[hi], hi, code)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def fp8_decode(bits: np.ndarray) -> np.ndarray:
    """OCP e4m3 codes -> fp32 values (no NaN codes are produced by fp8_bits)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    v = _E4M3[np.minimum(b & 0x7F, 126)]
    return np.where(b & 0x80, -v, v).astype(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded to bf16 (returned as fp32 holding bf16 values)."""
    return (bf16_bits(a).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class LayerSpec:
    name: str
    out_modes: tuple
    in_modes: tuple
    rank: int
    in_first: bool = False
    chain_perm: tuple | None = None  # chain position of each mode (outputs, then inputs)

    @property
    def n_out(self) -> int:
        return int(np.prod(self.out_modes))

    @property
    def n_in(self) -> int:
        return int(np.prod(self.in_modes))

    @property
    def chain_modes(self) -> list:
        if self.chain_perm is not None:
            listed = list(self.out_modes) + list(self.in_modes)
            modes = [0] * len(listed)
            for m, k in enumerate(self.chain_perm):
                modes[k] = listed[m]
            return modes
        if self.in_first:
            return list(self.in_modes) + list(self.out_modes)
        return list(self.out_modes) + list(self.in_modes)

    @property
    def split(self) -> int:
        """Chain link between the output and the input modes (cores before it)."""
        if self.chain_perm is not None:
            first_out = min(self.chain_perm[: len(self.out_modes)])
            return len(self.out_modes) if first_out == 0 else len(self.in_modes)
        return len(self.in_modes) if self.in_first else len(self.out_modes)

    @property
    def ranks(self) -> list:
        d = len(self.out_modes) + len(self.in_modes)
        return [1] + [int(self.rank)] * (d - 1) + [1]


def _six_layers(d_model_modes, ffn_modes, rank):
    return [
        LayerSpec("q", d_model_modes, d_model_modes, rank),
        LayerSpec("k", d_model_modes, d_model_modes, rank),
        LayerSpec("v", d_model_modes, d_model_modes, rank),
        LayerSpec("o", d_model_modes, d_model_modes, rank),
        LayerSpec("ffn1", ffn_modes, d_model_modes, rank),
        LayerSpec("ffn2", d_model_modes, ffn_modes, rank),
    ]


# tokens per step of each configuration
CONFIG_TOKENS = {0: 64, 1: 32 * 128, 2: 128 * 128, 3: 16384, 4: 64 * 256}
# fraction of each link's diagonal set to exactly zero
CONFIG_ZERO_FRAC = {0: 0.25, 1: 0.25, 2: 0.40, 4: 0.50}
CONFIG_DTYPE = {0: "f32", 1: "f32", 2: "bf16", 4: "bf16"}


def config_layers(config: int, rank: int | None = None) -> list:
    """The TT-linear layers of a configuration, in execution order."""
    if config == 0:
        return [LayerSpec("single", (12, 8, 8), (12, 8, 8), 12)]
    if config == 1:
        return _six_layers((12, 8, 8), (12, 16, 16), 30 if rank is None else rank)
    if config == 2:
        return _six_layers((12, 8, 8), (12, 16, 16), 30 if rank is None else rank)
    if config == 4:
        one = _six_layers((16, 8, 8), (16, 16, 16), 64 if rank is None else rank)
        return [LayerSpec(f"l{i}.{s.name}", s.out_modes, s.in_modes, s.rank) for i in range(24) for s in one]
    raise ValueError(f"configuration {config} has no TT-linear layers")


def make_link_diagonals(config, layer, ranks, zero_frac, base=BASE_SEED):
    rv = _rng(config, layer, _T_DVAL, base)
    rz = _rng(config, layer, _T_DZERO, base)
    D = []
    for r in ranks[1:-1]:
        v = rv.uniform(0.5, 1.5, r)
        nz = int(np.floor(zero_frac * r))
        v[rz.permutation(r)[:nz]] = 0.0
        D.append(v.astype(np.float32))
    return D


def make_tt_layer(config: int, layer: int, spec: LayerSpec, T: int, zero_frac: float,
                  dtype: str = "f32", base: int = BASE_SEED, acts: bool = True) -> dict:
    """Cores, link diagonals and activations of one TT-linear layer.

    Returns a dict with fp32 ``cores`` (r_{k-1}, n_k, r_k), fp32 ``D``
    (d-1 vectors), and when ``acts``: ``x`` (T x N_in) and ``dy`` (T x N_out)
    as fp32 arrays holding values exactly representable in ``dtype``, plus
    ``x_bits`` / ``dy_bits`` (uint16) for bf16.
    """
    ranks = spec.ranks
    modes = spec.chain_modes
    d = len(modes)
    D = make_link_diagonals(config, layer, ranks, zero_frac, base)
    prod_sq = float(np.prod([np.sum(v.astype(np.float64) ** 2) for v in D])) if D else 1.0
    if prod_sq == 0.0:
        prod_sq = 1.0
    sigma = (spec.n_in * prod_sq) ** (-1.0 / (2 * d))
    rc = _rng(config, layer, _T_CORES, base)
    cores = [(rc.standard_normal((ranks[k], modes[k], ranks[k + 1])) * sigma).astype(np.float32)
             for k in range(d)]
    out = {"spec": spec, "cores": cores, "D": D, "sigma": sigma, "T": T, "dtype": dtype,
           "seed": [config, layer, base]}
    if acts:
        x = _rng(config, layer, _T_X, base).standard_normal((T, spec.n_in), dtype=np.float32)
        dy = _rng(config, layer, _T_DY, base).standard_normal((T, spec.n_out), dtype=np.float32)
        if dtype == "bf16":
            out["x_bits"] = bf16_bits(x)
            out["dy_bits"] = bf16_bits(dy)
            x = (out["x_bits"].astype(np.uint32) << np.uint32(16)).view(np.float32)
            dy = (out["dy_bits"].astype(np.uint32) << np.uint32(16)).view(np.float32)
        elif dtype == "fp8":
            out["x_bits"] = fp8_bits(x)
            out["dy_bits"] = fp8_bits(dy)
            x = fp8_decode(out["x_bits"])
            dy = fp8_decode(out["dy_bits"])
        out["x"], out["dy"] = x, dy
    return out


@dataclass(frozen=True)
class TTMSpec:
    vocab_modes: tuple = (32, 32, 32)
    dim_modes: tuple = (12, 8, 8)
    ranks: tuple = (1, 16, 16, 1)

    @property
    def vocab(self) -> int:
        return int(np.prod(self.vocab_modes))

    @property
    def dim(self) -> int:
        return int(np.prod(self.dim_modes))


def zipf_ids(rng: np.random.Generator, T: int, vocab: int, s: float = 1.1) -> np.ndarray:
    p = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    ids = np.searchsorted(cdf, rng.random(T), side="right")
    return np.minimum(ids, vocab - 1).astype(np.int64)


def make_ttm(config: int = 3, spec: TTMSpec = TTMSpec(), T: int = 16384, std: float = 0.1,
             zipf_s: float = 1.1, with_D: bool = False, zero_frac: float = 0.25,
             base: int = BASE_SEED) -> dict:
    """TTM cores F_k (r, m, n, r') ~ N(0, std^2) fp32, Zipf ids, N(0,1) row grads."""
    rc = _rng(config, 0, _T_CORES, base)
    d = len(spec.vocab_modes)
    cores = [(rc.standard_normal((spec.ranks[k], spec.vocab_modes[k], spec.dim_modes[k], spec.ranks[k + 1]))
              * std).astype(np.float32) for k in range(d)]
    D = make_link_diagonals(config, 0, list(spec.ranks), zero_frac, base) if with_D else None
    ids = zipf_ids(_rng(config, 0, _T_IDS, base), T, spec.vocab, zipf_s)
    dout = _rng(config, 0, _T_DY, base).standard_normal((T, spec.dim), dtype=np.float32)
    return {"spec": spec, "cores": cores, "D": D, "ids": ids, "dout": dout, "T": T,
            "seed": [config, 0, base]}
