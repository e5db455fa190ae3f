"""The parity checker's own rules, exercised on the CPU with results that
the oracle itself produced (test infrastructure; no GPU involved)."""
import numpy as np
import torch

import oracle.layer as OL
import synth
from oracle.codec import bf16_encode, e4m3_encode
from tests.conftest import oracle_inputs
from oracle.codec import e4m3_decode as dec, e4m3_encode as enc
from tests.parity import check_layer, h_compare

WL = synth.Workload("rules_fp8", m=12, hidden=256, experts=6, topk=2, inter=256,
                    shared_inter=128, dtype="fp8", gating="sigmoid", routed_scale=2.5,
                    seed=50, shared_gate=True)


def _as_gpu(wl, inp):
    """Outputs and stage buffers shaped like the GPU's, from the oracle."""
    spec, args = oracle_inputs(wl, inp)
    r = OL.forward(spec, **args, keep_h=True)
    te = wl.m * wl.topk
    slot = r["slot_of_pair"]
    codes = np.zeros((te, wl.inter), np.uint8)
    scales = np.zeros((te, wl.inter // 128), np.float32)
    for p in range(te):
        s = r["h_scale"][p]
        codes[slot[p]] = e4m3_encode((r["h_pre"][p].astype(np.float32) /
                                      np.repeat(s, 128)).astype(np.float32))
        scales[slot[p]] = s
    sh_s = r["h_sh_scale"]
    sh_c = e4m3_encode((r["h_sh_pre"].astype(np.float32) /
                        np.repeat(sh_s, 128, axis=1)).astype(np.float32))
    out = torch.from_numpy(bf16_encode(r["out64"]).view(np.int16)).view(torch.bfloat16)
    dbg = {"h": torch.from_numpy(codes), "h_scale": torch.from_numpy(scales),
           "h_shared": torch.from_numpy(sh_c), "h_shared_scale": torch.from_numpy(sh_s),
           "slot_of_pair": torch.from_numpy(slot.astype(np.int32)),
           "sorted_pair": torch.from_numpy(r["sorted_pair"].astype(np.int32)),
           "counts": torch.from_numpy(r["counts"].astype(np.int32)),
           "offsets": torch.from_numpy(r["offsets"].astype(np.int32))}
    idx = torch.from_numpy(r["idx"].astype(np.int32))
    w = torch.from_numpy(r["w"].astype(np.float32))
    return out, idx, w, dbg


def test_oracle_results_pass_and_h_codes_are_checked():
    inp = synth.make_inputs(WL)
    out, idx, w, dbg = _as_gpu(WL, inp)
    rep = check_layer(WL, inp, out, idx, w, debug=dbg)
    assert rep.ok(), rep.failures
    assert rep.h_checked == WL.m * WL.topk * WL.inter + WL.m * WL.shared_inter
    assert rep.h_ties == 0 and rep.h_hard == 0


def test_a_code_off_away_from_a_tie_is_hard():
    inp = synth.make_inputs(WL)
    out, idx, w, dbg = _as_gpu(WL, inp)
    c = dbg["h"].numpy()
    c[3, 5] = (int(c[3, 5]) & 0x80) | min((int(c[3, 5]) & 0x7F) + 3, 0x7E)
    rep = check_layer(WL, inp, out, idx, w, debug=dbg)
    assert rep.h_hard == 1 and rep.h_ties == 0


def test_the_other_code_at_a_planted_tie_is_a_choice():
    """An h value placed exactly between two codes: the GPU's other code is
    accepted as a tie and the output compared with the oracle rerun with it;
    the same code flip away from a tie is not."""
    inp = synth.make_inputs(WL)
    spec, args = oracle_inputs(WL, inp)
    r = OL.forward(spec, **args, keep_h=True)
    p = 7
    s = float(r["h_scale"][p][0])
    pre = r["h_pre"][p].copy()
    col = int(np.argmax(np.abs(pre[:128]) < 0.5 * np.abs(pre[:128]).max()))
    q = pre[col] / s
    # the quotient's nearest code and the neighbour on the far side of it
    c0 = int(enc(np.float32(q)))
    v0 = float(dec(np.uint8(c0)))
    c1 = c0 + 1 if abs(q) > abs(v0) else c0 - 1
    v1 = float(dec(np.uint8(c1)))
    # move the exact value onto the midpoint: both codes are then correct
    pre_t = pre.copy()[None, :]
    pre_t[0, col] = 0.5 * (v0 + v1) * s
    gcodes = enc((r["h"][p] / np.repeat(r["h_scale"][p], 128)).astype(np.float32))[None, :]
    gcodes[0, col] = c1
    _, ties, hard = h_compare(pre_t, r["h"][p][None, :], r["h_scale"][p][None, :], gcodes,
                              r["h_scale"][p][None, :])
    assert len(ties) == 1 and hard == 0 and ties[0][:2] == (0, col)
    # the same choice with the exact value a tenth of a step from the midpoint
    pre_t[0, col] = (0.5 * (v0 + v1) + 0.1 * (v0 - v1)) * s
    _, ties, hard = h_compare(pre_t, r["h"][p][None, :], r["h_scale"][p][None, :], gcodes,
                              r["h_scale"][p][None, :])
    assert len(ties) == 0 and hard == 1


def test_a_wrong_scale_fails():
    inp = synth.make_inputs(WL)
    out, idx, w, dbg = _as_gpu(WL, inp)
    dbg["h_shared_scale"].numpy()[2, 0] *= 1.01
    rep = check_layer(WL, inp, out, idx, w, debug=dbg)
    assert any("h scale error" in f for f in rep.failures)


def test_a_wrong_output_fails():
    inp = synth.make_inputs(WL)
    out, idx, w, dbg = _as_gpu(WL, inp)
    o = out.float()
    o[4, 9] += 0.1 * float(o.abs().max())
    rep = check_layer(WL, inp, o.to(torch.bfloat16), idx, w, debug=dbg)
    assert not rep.ok()


def test_a_small_error_at_a_cancelling_output_fails():
    """The relative error is floored at a tenth of the output rms, not at the
    rms: an error of 5 % of 0.1 rms at an output below 0.1 rms fails the fp8
    bound (4e-2) although it is only 0.5 % of the rms."""
    inp = synth.make_inputs(WL)
    out, idx, w, dbg = _as_gpu(WL, inp)
    spec, args = oracle_inputs(WL, inp)
    r = OL.forward(spec, **args)["out64"]
    rms = float(np.sqrt(np.mean(r ** 2)))
    t, c = np.unravel_index(np.argmin(np.abs(r)), r.shape)
    o = torch.from_numpy(r).clone()
    o[t, c] = r[t, c] + 0.05 * 0.1 * rms
    rep = check_layer(WL, inp, o.float(), idx, w)
    assert rep.out_err_rms < 4e-2 < rep.out_err
    assert any("output error" in f for f in rep.failures)
