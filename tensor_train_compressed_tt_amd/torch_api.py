"""Torch-tensor front end of libttc: checks shapes, allocates the caller-owned
buffers with torch and passes device addresses and the current HIP stream to
the C entry points.  No arithmetic happens here."""

from __future__ import annotations

import math

import torch

from . import (
    TTC_BF16,
    TTC_F32,
    TTC_FP8,
    TTC_FLAG_PREPARED,
    TTC_PATH_AUTO,
    make_linear_desc,
    make_ttm_desc,
    tt_linear_bwd_cores,
    tt_linear_bwd_cores_batch,
    tt_linear_bwd_data,
    tt_linear_bwd_data_batch,
    tt_linear_bwd_split,
    tt_linear_fwd,
    tt_linear_fwd_batch,
    tt_linear_prepare,
    tt_linear_prepare_batch,
    tt_linear_rank_grads,
    tt_linear_rank_grads_batch,
    tt_linear_workspace,
    ttm_embed_bwd,
    ttm_embed_fwd,
    ttm_embed_index,
    ttm_embed_lookup,
    ttm_embed_workspace,
)

_ACT = {torch.float32: TTC_F32, torch.bfloat16: TTC_BF16, torch.float8_e4m3fn: TTC_FP8}


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need_buf(t: torch.Tensor, name: str):
    """A caller-supplied workspace: any contiguous device tensor; its size in
    bytes is what the C entry points receive."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def _need_grads(dG, shapes, name="dG"):
    if len(dG) != len(shapes):
        raise ValueError(f"{name} needs {len(shapes)} tensors, got {len(dG)}")
    for k, (g, s) in enumerate(zip(dG, shapes)):
        _need(g, f"{name}[{k}]", torch.float32, s)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class TTLinear:
    """A TT-linear layer y = x W^T with W given by cores and link diagonals.

    ``ranks`` lists r_0..r_d in chain order (output modes first unless
    ``in_first``).  Cores are fp32 (r_{k-1}, n_k, r_k); D is a list of d-1 fp32
    vectors; activations are fp32 or bf16.
    """

    def __init__(self, out_modes, in_modes, ranks, dtype=torch.float32, in_first=False, path=TTC_PATH_AUTO,
                 chain_perm=None):
        self.out_modes = tuple(int(n) for n in out_modes)
        self.in_modes = tuple(int(n) for n in in_modes)
        self.ranks = tuple(int(r) for r in ranks)
        self.in_first = bool(in_first)
        self.chain_perm = None if chain_perm is None else tuple(int(k) for k in chain_perm)
        self.dtype = dtype
        self.n_out = math.prod(self.out_modes)
        self.n_in = math.prod(self.in_modes)
        self.desc = make_linear_desc(self.out_modes, self.in_modes, self.ranks, _ACT[dtype], in_first, path,
                                     chain_perm=self.chain_perm)
        self.desc_prepared = make_linear_desc(self.out_modes, self.in_modes, self.ranks, _ACT[dtype], in_first, path,
                                              TTC_FLAG_PREPARED, chain_perm=self.chain_perm)
        listed = list(self.out_modes) + list(self.in_modes)
        if self.chain_perm is not None:
            modes = [0] * len(listed)
            for m, k in enumerate(self.chain_perm):
                modes[k] = listed[m]
        elif in_first:
            modes = list(self.in_modes) + list(self.out_modes)
        else:
            modes = listed
        self.core_shapes = [(self.ranks[k], modes[k], self.ranks[k + 1]) for k in range(len(modes))]

    def workspace(self, T: int):
        return tt_linear_workspace(self.desc, T)

    def alloc(self, T: int, device="cuda"):
        """Fresh (saved, scratch) byte buffers for T tokens."""
        sb, cb = self.workspace(T)
        return (torch.empty(max(sb, 256), dtype=torch.uint8, device=device),
                torch.empty(max(cb, 256), dtype=torch.uint8, device=device))

    def _check_chain(self, cores, D):
        if len(cores) != len(self.core_shapes) or len(D) != len(self.core_shapes) - 1:
            raise ValueError("wrong number of cores / diagonals")
        for k, (c, s) in enumerate(zip(cores, self.core_shapes)):
            _need(c, f"core {k}", torch.float32, s)
        for k, v in enumerate(D):
            _need(v, f"D {k}", torch.float32, (self.core_shapes[k][2],))

    def prepare(self, T, cores, D, saved=None):
        """Merge the cores into `saved` on the current stream (see tt_linear_prepare)."""
        self._check_chain(cores, D)
        sb, _ = self.workspace(T)
        if saved is None:
            saved = torch.empty(max(sb, 256), dtype=torch.uint8, device=cores[0].device)
        tt_linear_prepare(self.desc, T, [c.data_ptr() for c in cores], [v.data_ptr() for v in D], saved.data_ptr(),
                          _nbytes(saved), _stream())
        return saved

    def forward(self, x, cores, D, out=None, saved=None, prepared=False):
        T = int(x.shape[0])
        _need(x, "x", self.dtype, (T, self.n_in))
        self._check_chain(cores, D)
        if out is None:
            out = torch.empty((T, self.n_out), dtype=self.dtype, device=x.device)
        _need(out, "out", self.dtype, (T, self.n_out))
        sb, _ = self.workspace(T)
        if saved is None:
            if prepared:
                raise ValueError("prepared=True needs the saved buffer filled by prepare()")
            saved = torch.empty(max(sb, 256), dtype=torch.uint8, device=x.device)
        desc = self.desc_prepared if prepared else self.desc
        tt_linear_fwd(desc, T, x.data_ptr(), [c.data_ptr() for c in cores], [v.data_ptr() for v in D],
                      out.data_ptr(), saved.data_ptr(), _nbytes(saved), None, 0, _stream())
        return out, saved

    def backward(self, x, dy, cores, D, saved, want_dx=True, dx=None, dG=None, scratch=None, grad_stream=None):
        """dX on the current stream; dG on `grad_stream` (a torch.cuda.Stream) when given."""
        T = int(x.shape[0])
        _need(x, "x", self.dtype, (T, self.n_in))
        _need(dy, "dy", self.dtype, (T, self.n_out))
        self._check_chain(cores, D)
        _need_buf(saved, "saved")
        _, cb = self.workspace(T)
        own_scratch = scratch is None
        if own_scratch:
            scratch = torch.empty(max(cb, 256), dtype=torch.uint8, device=x.device)
        _need_buf(scratch, "scratch")
        if want_dx:
            if dx is None:
                dx = torch.empty((T, self.n_in), dtype=self.dtype, device=x.device)
            _need(dx, "dx", self.dtype, (T, self.n_in))
        own_dG = dG is None
        if own_dG:
            dG = [torch.empty(s, dtype=torch.float32, device=x.device) for s in self.core_shapes]
        _need_grads(dG, self.core_shapes)
        main = _stream()
        gs = main if grad_stream is None else grad_stream.cuda_stream
        tt_linear_bwd_split(self.desc, T, x.data_ptr(), dy.data_ptr(), [c.data_ptr() for c in cores],
                            [v.data_ptr() for v in D], saved.data_ptr(), _nbytes(saved),
                            dx.data_ptr() if want_dx else None, [g.data_ptr() for g in dG], scratch.data_ptr(),
                            _nbytes(scratch), main, gs)
        if grad_stream is not None and gs != main:
            # the core-gradient tail on grad_stream still reads scratch and
            # writes dG after this call returns: keep the allocator from
            # handing their blocks to work on the current stream before then
            if own_scratch:
                scratch.record_stream(grad_stream)
            if own_dG:
                for g in dG:
                    g.record_stream(grad_stream)
        return (dx if want_dx else None), dG


    def backward_data(self, x, dy, cores, D, saved, scratch, want_dx=True, dx=None):
        """dX on the current stream; the partial sums for backward_cores stay in `scratch`."""
        T = int(x.shape[0])
        _need(x, "x", self.dtype, (T, self.n_in))
        _need(dy, "dy", self.dtype, (T, self.n_out))
        self._check_chain(cores, D)
        _need_buf(saved, "saved")
        _need_buf(scratch, "scratch")
        if want_dx:
            if dx is None:
                dx = torch.empty((T, self.n_in), dtype=self.dtype, device=x.device)
            _need(dx, "dx", self.dtype, (T, self.n_in))
        tt_linear_bwd_data(self.desc, T, x.data_ptr(), dy.data_ptr(), [c.data_ptr() for c in cores],
                           [v.data_ptr() for v in D], saved.data_ptr(), _nbytes(saved),
                           dx.data_ptr() if want_dx else None, scratch.data_ptr(), _nbytes(scratch), _stream())
        return dx if want_dx else None

    def backward_cores(self, T, cores, D, saved, scratch, dG=None):
        """dG on the current stream from the partial sums backward_data left in `scratch`."""
        self._check_chain(cores, D)
        _need_buf(saved, "saved")
        _need_buf(scratch, "scratch")
        if dG is None:
            dG = [torch.empty(s, dtype=torch.float32, device=cores[0].device) for s in self.core_shapes]
        _need_grads(dG, self.core_shapes)
        tt_linear_bwd_cores(self.desc, int(T), [c.data_ptr() for c in cores], [v.data_ptr() for v in D],
                            saved.data_ptr(), _nbytes(saved), [g.data_ptr() for g in dG], scratch.data_ptr(),
                            _nbytes(scratch), _stream())
        return dG

    def rank_grads(self, cores, D, dG, gamma=0.0, beta=0.0, dD=None):
        """Early-stage gradients on the current stream: returns dD (one fp32
        vector per link) and adds 2 beta G_k to dG in place (see
        tt_linear_rank_grads)."""
        self._check_chain(cores, D)
        _need_grads(dG, self.core_shapes)
        if dD is None:
            dD = [torch.empty(v.shape, dtype=torch.float32, device=v.device) for v in D]
        tt_linear_rank_grads(self.desc, [c.data_ptr() for c in cores], [v.data_ptr() for v in D],
                             [g.data_ptr() for g in dG], [v.data_ptr() for v in dD], gamma, beta, _stream())
        return dD

def prepare_batch(mods, T, cores, D, saved):
    """TTLinear.prepare for several layers in one batched call on the current
    stream (lists with one entry per layer; `saved` buffers are required)."""
    for m, c, d in zip(mods, cores, D):
        m._check_chain(c, d)
    tt_linear_prepare_batch([m.desc for m in mods], [T] * len(mods),
                            [[t.data_ptr() for t in c] for c in cores], [[v.data_ptr() for v in d] for d in D],
                            [b.data_ptr() for b in saved], [_nbytes(b) for b in saved], _stream())



def forward_batch(mods, xs, cores, D, outs, saved, prepared=False):
    """TTLinear.forward of several independent layers in one batched call on
    the current stream (lists with one entry per layer; outputs and saved
    buffers are required)."""
    for m, x, c, d, y in zip(mods, xs, cores, D, outs):
        T = int(x.shape[0])
        _need(x, "x", m.dtype, (T, m.n_in))
        _need(y, "out", m.dtype, (T, m.n_out))
        m._check_chain(c, d)
    tt_linear_fwd_batch([m.desc_prepared if prepared else m.desc for m in mods], [int(x.shape[0]) for x in xs],
                        [x.data_ptr() for x in xs], [[t.data_ptr() for t in c] for c in cores],
                        [[v.data_ptr() for v in d] for d in D], [y.data_ptr() for y in outs],
                        [b.data_ptr() for b in saved], [_nbytes(b) for b in saved], _stream())


def backward_data_batch(mods, xs, dys, cores, D, saved, scratch, dxs):
    """TTLinear.backward_data of several independent layers in one batched
    call on the current stream; dxs entries may be None (dX skipped)."""
    for m, x, dy, c, d in zip(mods, xs, dys, cores, D):
        T = int(x.shape[0])
        _need(x, "x", m.dtype, (T, m.n_in))
        _need(dy, "dy", m.dtype, (T, m.n_out))
        m._check_chain(c, d)
    for m, x, dx in zip(mods, xs, dxs):
        if dx is not None:
            _need(dx, "dx", m.dtype, (int(x.shape[0]), m.n_in))
    for b in list(saved) + list(scratch):
        _need_buf(b, "saved/scratch")
    tt_linear_bwd_data_batch([m.desc for m in mods], [int(x.shape[0]) for x in xs], [x.data_ptr() for x in xs],
                             [dy.data_ptr() for dy in dys], [[t.data_ptr() for t in c] for c in cores],
                             [[v.data_ptr() for v in d] for d in D], [b.data_ptr() for b in saved],
                             [_nbytes(b) for b in saved], [None if t is None else t.data_ptr() for t in dxs],
                             [b.data_ptr() for b in scratch], [_nbytes(b) for b in scratch], _stream())

def backward_cores_batch(mods, T, cores, D, saved, scratch, dG):
    """TTLinear.backward_cores for several layers in one batched call on the
    current stream; each layer's backward_data must have run before."""
    for m, c, d, g in zip(mods, cores, D, dG):
        m._check_chain(c, d)
        _need_grads(g, m.core_shapes)
    for b in list(saved) + list(scratch):
        _need_buf(b, "saved/scratch")
    tt_linear_bwd_cores_batch([m.desc for m in mods], [T] * len(mods),
                              [[t.data_ptr() for t in c] for c in cores], [[v.data_ptr() for v in d] for d in D],
                              [b.data_ptr() for b in saved], [_nbytes(b) for b in saved],
                              [[g.data_ptr() for g in gl] for gl in dG],
                              [b.data_ptr() for b in scratch], [_nbytes(b) for b in scratch], _stream())

class TTMEmbedding:
    """A TTM embedding table: cores F_k (r_{k-1}, m_k, n_k, r_k) fp32."""

    def __init__(self, vocab_modes, dim_modes, ranks, mode=0):
        self.vocab_modes = tuple(int(n) for n in vocab_modes)
        self.dim_modes = tuple(int(n) for n in dim_modes)
        self.ranks = tuple(int(r) for r in ranks)
        self.vocab = math.prod(self.vocab_modes)
        self.dim = math.prod(self.dim_modes)
        self.core_shapes = [(self.ranks[k], self.vocab_modes[k], self.dim_modes[k], self.ranks[k + 1])
                            for k in range(len(self.vocab_modes))]
        self.mode = int(mode)  # TTC_TTM_DEDUP / _UNIQUE / _PLAIN

    def desc(self, accumulate=False):
        return make_ttm_desc(self.vocab_modes, self.dim_modes, self.ranks, accumulate, self.mode)

    def workspace(self, T: int):
        return ttm_embed_workspace(self.desc(), T)

    def _check(self, cores, D):
        if len(cores) != len(self.core_shapes):
            raise ValueError("wrong number of cores")
        for k, (c, s) in enumerate(zip(cores, self.core_shapes)):
            _need(c, f"core {k}", torch.float32, s)
        if D is not None:
            for k, v in enumerate(D):
                _need(v, f"D {k}", torch.float32, (self.ranks[k + 1],))

    def forward(self, ids, cores, D=None, out=None, saved=None, scratch=None):
        T = int(ids.shape[0])
        _need(ids, "ids", torch.int64, (T,))
        self._check(cores, D)
        sb, cb = self.workspace(T)
        if out is None:
            out = torch.empty((T, self.dim), dtype=torch.float32, device=ids.device)
        _need(out, "out", torch.float32, (T, self.dim))
        if saved is None:
            saved = torch.empty(max(sb, 256), dtype=torch.uint8, device=ids.device)
        if scratch is None:
            scratch = torch.empty(max(cb, 256), dtype=torch.uint8, device=ids.device)
        _need_buf(saved, "saved")
        _need_buf(scratch, "scratch")
        ttm_embed_fwd(self.desc(), T, ids.data_ptr(), [c.data_ptr() for c in cores],
                      None if D is None else [v.data_ptr() for v in D], out.data_ptr(), saved.data_ptr(),
                      _nbytes(saved), scratch.data_ptr(), _nbytes(scratch), _stream())
        return out, saved

    def index(self, ids, saved=None):
        """The index of a lookup of `ids` into `saved` on the current stream
        (see ttm_embed_index); returns saved."""
        T = int(ids.shape[0])
        _need(ids, "ids", torch.int64, (T,))
        sb, _ = self.workspace(T)
        if saved is None:
            saved = torch.empty(max(sb, 256), dtype=torch.uint8, device=ids.device)
        ttm_embed_index(self.desc(), T, ids.data_ptr(), saved.data_ptr(), _nbytes(saved), _stream())
        return saved

    def lookup(self, T, cores, D, saved, out=None, scratch=None):
        """The rows of the lookup whose index `saved` holds (see ttm_embed_lookup)."""
        self._check(cores, D)
        _, cb = self.workspace(T)
        dev = cores[0].device
        if out is None:
            out = torch.empty((T, self.dim), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, (int(T), self.dim))
        if scratch is None:
            scratch = torch.empty(max(cb, 256), dtype=torch.uint8, device=dev)
        _need_buf(saved, "saved")
        _need_buf(scratch, "scratch")
        ttm_embed_lookup(self.desc(), int(T), [c.data_ptr() for c in cores],
                         None if D is None else [v.data_ptr() for v in D], out.data_ptr(), saved.data_ptr(),
                         _nbytes(saved), scratch.data_ptr(), _nbytes(scratch), _stream())
        return out

    def backward(self, ids, dout, cores, D, saved, dF=None, accumulate=False, scratch=None):
        T = int(ids.shape[0])
        _need(ids, "ids", torch.int64, (T,))
        _need(dout, "dout", torch.float32, (T, self.dim))
        self._check(cores, D)
        _, cb = self.workspace(T)
        if scratch is None:
            scratch = torch.empty(max(cb, 256), dtype=torch.uint8, device=ids.device)
        if dF is None:
            dF = [torch.empty(s, dtype=torch.float32, device=ids.device) for s in self.core_shapes]
        _need_grads(dF, self.core_shapes, "dF")
        _need_buf(saved, "saved")
        _need_buf(scratch, "scratch")
        ttm_embed_bwd(self.desc(accumulate), T, ids.data_ptr(), dout.data_ptr(), [c.data_ptr() for c in cores],
                      None if D is None else [v.data_ptr() for v in D], saved.data_ptr(), _nbytes(saved),
                      [g.data_ptr() for g in dF], scratch.data_ptr(), _nbytes(scratch), _stream())
        return dF


def rank_grads_batch(mods, cores, D, dG, dD, gamma=0.0, beta=0.0):
    """TTLinear.rank_grads for several layers in one launch on the current stream."""
    for m, c, d, g, dd in zip(mods, cores, D, dG, dD):
        m._check_chain(c, d)
        _need_grads(g, m.core_shapes)
        _need_grads(dd, [(s[2],) for s in m.core_shapes[:-1]], "dD")
    tt_linear_rank_grads_batch([m.desc for m in mods], [[t.data_ptr() for t in c] for c in cores],
                               [[v.data_ptr() for v in d] for d in D], [[t.data_ptr() for t in g] for g in dG],
                               [[v.data_ptr() for v in dd] for dd in dD], gamma, beta, _stream())
