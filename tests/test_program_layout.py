"""Host-side layout of a Copy-as-Decode program (no GPU): the forwards the op schedule expands
to (Copy-as-Decode §2.3 step types, Appendix A states and token identifiers) and the device
buffers the program runner builds from them."""
import numpy as np
import torch

from spec_verify_cad_amd import cad, synth
from spec_verify_cad_amd.configs import CONFIGS, QWEN7, cad_program_inputs
from spec_verify_cad_amd.program import DeviceProgram

T = synth.CAD_TOK


def test_token_ids_of_the_literals():
    # the byte-order reading puts "<" and ">" where the page's table has them
    assert synth._char_id("<") == T["LT"] and synth._char_id(">") == T["GT"]
    assert synth.CAD_DIGITS == tuple(range(15, 25))


def test_copy_op_expansion():
    f = synth.cad_program_forwards([("copy", 95, 30)], line_tokens=10)
    # "<" -> op type; forced (copy, lines, =") -> first digit; "10-13" one char per forward; splice
    assert [x.role for x in f] == ["op_type", "copy_open"] + ["line_char"] * 5 + ["splice", "close"]
    chars = "".join(chr(x.lits[0] + 33) for x in f if x.role == "line_char")
    assert chars == "10-13"
    lc = [x.allowed for x in f if x.role == "line_char"]
    assert lc[0] == synth.CAD_DIGITS + (synth.CAD_HYPHEN,)          # after "1": digit or "-"
    assert lc[2] == synth.CAD_DIGITS                                 # after "-": a digit
    assert lc[4] == synth.CAD_DIGITS + (synth.CAD_QUOTE,)            # after "3": digit or closing quote
    sp = f[-2]
    assert sp.lits == (synth.CAD_QUOTE, T["SLASH_GT"]) and sp.doc == (95, 30) and sp.n == 32
    assert sp.allowed == (T["LT"], T["LT_SLASH"])
    assert f[-1].lits == (T["LT_SLASH"], T["PROGRAM"], T["GT"]) and f[-1].allowed is None


def test_gen_op_expansion():
    f = synth.cad_program_forwards([("gen", 3)])
    assert [x.role for x in f] == ["op_type", "gen_open", "gen_body", "gen_body", "gen_body",
                                   "gen_close", "gen_close", "gen_close", "close"]
    assert f[1].lits == (T["GEN"], T["GT"]) and f[1].allowed is None
    assert all(x.from_prev and x.n == 1 for x in f[2:5])
    assert [x.lits[0] for x in f[5:8]] == [T["LT_SLASH"], T["GEN"], T["GT"]]
    assert f[7].allowed == (T["LT"], T["LT_SLASH"])


def test_program_schedule_properties():
    doc, ops = cad_program_inputs(CONFIGS["qwen7_cad_program"])
    f = synth.cad_program_forwards(ops)
    out = sum(o[2] if o[0] == "copy" else o[1] for o in ops)
    assert out == CONFIGS["qwen7_cad_program"].extra["total_out"]
    # content = copied + generated tokens; everything else fed is grammar structure
    content = sum(x.doc[1] for x in f if x.doc) + sum(1 for x in f if x.role == "gen_body")
    assert content == out
    assert all(len(x.allowed) <= 12 for x in f if x.allowed)       # at most 12 ids at a masked step
    assert sum(1 for x in f if x.role == "op_type") == len(ops)


def test_device_program_buffers_on_the_host():
    doc = np.arange(1000, 1100, dtype=np.int32)
    ops = [("copy", 5, 4), ("gen", 2)]
    fwds = synth.cad_program_forwards(ops, line_tokens=10)
    shp = QWEN7
    tens = {n: torch.zeros(1, dtype=torch.int16) for n in synth.weight_shapes(shp)}
    lay = cad.DeviceLayer.from_tensors(shp, tens)
    cache = cad.DeviceCache(shp, 1, 64, device="cpu")
    prog = DeviceProgram(lay, cache, doc, fwds, device="cpu")
    assert prog.fed == sum(x.n for x in fwds)
    assert prog.workspace.numel() >= cad.span_forward_workspace(lay, 1, 6, cad.MASK_CAUSAL, 1, 1, 64,
                                                                cad.COMMIT_ALL | cad.LOGITS_LAST)
    for f, x in enumerate(fwds):
        if x.allowed:
            row = prog.allowed[f].numpy()
            assert list(row[:len(x.allowed)]) == list(x.allowed) and (row[len(x.allowed):] == -1).all()
        if x.from_prev:
            assert prog.tok_off[f] == -1
    # splice tokens: quote, "/>", doc[5:9]
    sp = next(f for f, x in enumerate(fwds) if x.role == "splice")
    o = int(prog.tok_off[sp])
    assert list(prog.tokens[o:o + 6].numpy()) == [synth.CAD_QUOTE, T["SLASH_GT"], 1005, 1006, 1007, 1008]
    # the fed stream reads generated tokens from the previous forward's decision
    prog.decisions.copy_(torch.arange(len(fwds), dtype=torch.int32) + 7000)
    s = prog.fed_tokens(doc)
    assert len(s) == prog.fed
    gb = [f for f, x in enumerate(fwds) if x.role == "gen_body"]
    pos = [sum(x.n for x in fwds[:f]) for f in gb]
    assert [int(s[p]) for p in pos] == [7000 + f - 1 for f in gb]


def test_device_program_rejects_bad_layouts():
    import pytest
    shp = QWEN7
    tens = {n: torch.zeros(1, dtype=torch.int16) for n in synth.weight_shapes(shp)}
    lay = cad.DeviceLayer.from_tensors(shp, tens)
    doc = np.arange(10, dtype=np.int32)
    with pytest.raises(ValueError):                       # batch of two
        DeviceProgram(lay, cad.DeviceCache(shp, 2, 64, device="cpu"), doc, [], device="cpu")
    c1 = cad.DeviceCache(shp, 1, 64, device="cpu")
    with pytest.raises(ValueError):                       # nothing before the first fed-back token
        DeviceProgram(lay, c1, doc, [synth.ProgramForward("gen_body", from_prev=True)], device="cpu")
    with pytest.raises(ValueError):                       # more allowed ids than the kernel takes
        DeviceProgram(lay, c1, doc, [synth.ProgramForward("x", (1,), allowed=tuple(range(cad.MAX_ALLOWED + 1)))],
                      device="cpu")
    with pytest.raises(ValueError):                       # a stack needs a stack cache
        DeviceProgram(cad.DeviceStack([lay, lay]), c1, doc, [], device="cpu")
