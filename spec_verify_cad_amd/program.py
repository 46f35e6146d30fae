"""A Copy-as-Decode program on the device: every forward of the program (masked decision steps,
forced-template prefills, copy splices and free generation, Copy-as-Decode §2.3 and §2.4) enqueued
back to back on one stream, with no host synchronisation between them.

Known input tokens (literals and document slices) are laid out once in one device buffer; a
generated token is read by the next forward straight from the slot the previous forward wrote,
so the host never waits for a decision.  All arithmetic runs in the library's kernels."""
from __future__ import annotations

import numpy as np
import torch

from . import cad
from .synth import ProgramForward


class DeviceProgram:
    """The forwards of one program for a batch-1 cache.

    decisions[f] receives the token forward f chose after its last row (masked forwards: the
    allowed id with the largest logit; the others: the unrestricted argmax)."""

    def __init__(self, layer, cache, doc: np.ndarray, forwards: list, device=None):
        """layer / cache: a DeviceLayer with its DeviceCache, or a DeviceStack with its StackCache
        (the program then runs through every layer)."""
        if cache.B != 1:
            raise ValueError("a program runs on a batch-1 cache")
        self.stacked = isinstance(layer, cad.DeviceStack)
        if self.stacked != isinstance(cache, cad.StackCache):
            raise ValueError("a stack runs on a stack cache")
        dev = device if device is not None else cache.len.device
        self.layer, self.cache, self.forwards = layer, cache, list(forwards)
        F = len(self.forwards)
        toks, self.tok_off = [], np.full(F, -1, dtype=np.int64)
        allowed = np.full((F, cad.MAX_ALLOWED), -1, dtype=np.int32)
        off = 0
        for f, pf in enumerate(self.forwards):
            if pf.allowed is not None:
                if not 1 <= len(pf.allowed) <= cad.MAX_ALLOWED:
                    raise ValueError(f"forward {f}: {len(pf.allowed)} allowed ids")
                allowed[f, :len(pf.allowed)] = pf.allowed
            if pf.from_prev:
                if f == 0:
                    raise ValueError("the first forward has no previous decision to read")
                continue
            t = list(pf.lits)
            if pf.doc is not None:
                s, n = pf.doc
                t += [int(x) for x in doc[s:s + n]]
            self.tok_off[f] = off
            toks += t
            off += len(t)
        self.tokens = torch.tensor(toks, dtype=torch.int32, device=dev)
        self.allowed = torch.from_numpy(allowed).to(dev)
        self.decisions = torch.full((F,), -1, dtype=torch.int32, device=dev)
        self.fed = sum(pf.n for pf in self.forwards)
        sizes = {}
        for pf in self.forwards:
            key = (pf.n, self._flags(pf))
            if key not in sizes:
                if self.stacked:
                    sizes[key] = cad.stack_span_forward_workspace(layer, 1, pf.n, cad.MASK_CAUSAL, 1, 1, cache.cap,
                                                                  key[1])
                else:
                    sizes[key] = cad.span_forward_workspace(layer, 1, pf.n, cad.MASK_CAUSAL, 1, 1, cache.cap, key[1])
        self.workspace = cad.alloc_workspace(max(sizes.values()), device=dev)

    @staticmethod
    def _flags(pf: ProgramForward) -> int:
        return cad.COMMIT_ALL | (cad.LOGITS_LAST if pf.n > 1 else 0)

    def enqueue(self, stream=None):
        """Enqueue every forward; the cache grows by `fed` rows."""
        for f in range(len(self.forwards)):
            self.enqueue_one(f, stream)

    def enqueue_one(self, f: int, stream=None):
        """Enqueue forward f (after forward f - 1, whose decision it may read)."""
        pf = self.forwards[f]
        n = pf.n
        if pf.from_prev:
            tok = self.decisions[f - 1:f].view(1, 1)
        else:
            o = int(self.tok_off[f])
            tok = self.tokens[o:o + n].view(1, n)
        out = self.decisions[f:f + 1]
        if pf.allowed is None:
            fwd = cad.stack_span_forward if self.stacked else cad.span_forward
            fwd(self.layer, self.cache, tok, n, flags=self._flags(pf), argmax_out=out, workspace=self.workspace,
                stream=stream)
        else:
            A = len(pf.allowed)
            fwd = cad.stack_span_forward_allowed if self.stacked else cad.span_forward_allowed
            fwd(self.layer, self.cache, tok, n, self.allowed[f:f + 1, :A], A, flags=self._flags(pf),
                argmax_out=out, workspace=self.workspace, stream=stream)

    def fed_tokens(self, doc: np.ndarray) -> np.ndarray:
        """The program's input stream in cache order (reads the decisions back: synchronises)."""
        dec = self.decisions.cpu().numpy()
        out = []
        for f, pf in enumerate(self.forwards):
            if pf.from_prev:
                out.append(int(dec[f - 1]))
            else:
                out += list(pf.lits)
                if pf.doc is not None:
                    s, n = pf.doc
                    out += [int(x) for x in doc[s:s + n]]
        return np.asarray(out, dtype=np.int32)
