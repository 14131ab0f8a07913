"""GPU parity of the DFlow relay (dflow_relay + relay-aware dflash_draft_block)
against the float64 oracle.

Workload: the relay configuration (tiny fp32 drafter with 5 tapped target
layers, B 16), 8 requests prefilled with 64 context tokens, then 64
draft-verify rounds with the accepted count of every request drawn from
U{0..15}.  Each round both sides follow the oracle's branch (targets are built
from the oracle's candidates), fuse the committed rows, and relay the reusable
rejected suffix.  Bars: relay rows and logits rel <= 1e-4 (fp32), top-1 ids
where the oracle's margin exceeds 0.05, acceptance bit-exact."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from oracle import dflow as ofl
from synth.configs import QWEN3_4B
from tests._gpu import GpuDraft, check_top1, hidden_rows, log, rel_inf

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _cat(parts, d):
    return [np.ascontiguousarray(np.concatenate([p[l] for p in parts], axis=0)) for l in range(d.L)]


class RelayRig:
    def __init__(self, d, seed, bs, max_ctx):
        import block_diffusion_drafter_fuse_amd as dfa
        self.dfa = dfa
        self.d = d
        self.seed = seed
        self.w_np = synth.make_weights(d, seed)
        self.rw_np = synth.make_relay_weights(d, seed)
        self.g = GpuDraft(d, self.w_np, max_ctx=max_ctx, max_slots=bs, max_batch=bs)
        self.rw_dev = {k: dfa.to_device(v) for k, v in self.rw_np.items()}
        self.w32 = synth.weights_as_f32(self.w_np)
        self.rw32 = {k: synth.as_f32([v])[0] for k, v in self.rw_np.items()}
        self.o = oracle.OracleDrafter(self.w32, d)
        self.state = ofl.RelayState()

    def relay(self, slots, n_acc, cand, bonus, suffix):
        """suffix: per request, L arrays [k_r, Dt] (storage dtype)."""
        d = self.d
        parts = [s for s in suffix if s[0].shape[0]]
        hid = [self.dfa.to_device(h) for h in _cat(parts, d)] if parts else [None] * d.L
        c = torch.tensor(np.ascontiguousarray(cand, dtype=np.int32), device="cuda")
        b = torch.tensor(np.ascontiguousarray(bonus, dtype=np.int32), device="cuda")
        self.g.dr.relay(slots, [int(n) for n in n_acc], c, 1, b, hid, self.rw_dev["w1"], self.rw_dev["w2"])
        torch.cuda.synchronize()
        for i, r in enumerate(slots):
            k = max(0, d.B - 2 - int(n_acc[i]))
            if k:
                x = ofl.relay_inputs(self.w32, d, self.rw32, synth.as_f32(suffix[i]), int(bonus[i]),
                                     int(cand[i][int(n_acc[i])]))
                self.state.set(r, int(n_acc[i]), d.B, x)
            else:
                self.state.take(r)

    def read_relay(self, slot):
        out = torch.zeros((self.d.B, self.d.D), dtype=torch.float32, device="cuda")
        n = self.g.dr.read_relay(slot, out)
        torch.cuda.synchronize()
        return n, out.cpu().numpy()


def test_gpu_relay_rounds():
    wl = synth.get_config("dflow_relay")
    d, bs, B = wl.dims, wl.bs, wl.dims.B
    log(f"case dflow relay: bs {bs}, B {B}, L {d.L}, {wl.rounds} rounds")
    rig = RelayRig(d, wl.seed, bs, max_ctx=wl.ctx[0] + wl.rounds * B + B)
    slots = list(range(bs))
    rig.g.fuse(slots, wl.n_new, hidden_rows(d, wl.seed, [(r, 0, wl.n_new[r]) for r in range(bs)]))
    for r in range(bs):
        rig.o.fuse(r, synth.as_f32(synth.make_hidden(d, wl.seed, r, 0, wl.n_new[r])))
    anchors = synth.make_anchors(d, wl.seed, bs)
    nacc = synth.draw_accepted(bs, wl.rounds, B, wl.seed)
    relayed_rows = 0
    for t in range(wl.rounds):
        # the GPU's stored relay rows equal the oracle's before they are used
        for r in slots:
            n, rows = rig.read_relay(r)
            want = rig.state.rows.get(r, {})
            assert n == len(want), f"round {t} req {r}: relay count {n} vs {len(want)}"
            for off, x in want.items():
                err = rel_inf(rows[off], x)
                assert err <= 1e-4, f"round {t} req {r} offset {off}: relay row rel err {err}"
            relayed_rows += n
        ids, _, lg = rig.g.draft(slots, anchors, top_k=1, logits=True)
        cand = np.zeros((bs, B - 1), np.int32)
        for r in slots:
            x0 = ofl.block_inputs(rig.w32, d, int(anchors[r]), rig.state.take(r))
            ref = oracle.draft_block(rig.w32, d, rig.o.cache(r), int(anchors[r]), x0)["logits"]
            err = rel_inf(lg[r], ref)
            assert err <= 1e-4, f"round {t} req {r}: logits rel err {err}"
            _, bad = check_top1(ids[r][:, 0], ref)
            assert len(bad) == 0, f"round {t} req {r}: top-1 mismatch at {bad}"
            cand[r] = oracle.topk(ref, 1)[0][:, 0]
        for r in slots:   # the draft consumed the relay
            assert rig.read_relay(r)[0] == 0
        m = nacc[t]
        tgt = synth.make_targets(cand, m, d.V, wl.seed * 1000 + t)
        tau, bonus = rig.g.accept(cand, 1, tgt)
        for r in slots:
            tr, br = oracle.accept(cand[r], tgt[r])
            assert (int(tau[r]), int(bonus[r])) == (tr, br) and tr == int(m[r]) + 1
        # commit: the anchor and the accepted candidates (tau rows) are fused
        pos0 = [rig.o.cache(r).length for r in slots]
        rows = hidden_rows(d, wl.seed, [(r, pos0[r], int(tau[r])) for r in slots])
        rig.g.fuse(slots, [int(x) for x in tau], rows)
        for r in slots:
            rig.o.fuse(r, synth.as_f32(synth.make_hidden(d, wl.seed, r, pos0[r], int(tau[r]))))
            assert rig.g.dr.slot_len(r) == rig.o.cache(r).length
        # relay of the reusable rejected suffix (skipped where none exists)
        suffix = [synth.make_suffix_hidden(d, wl.seed, r, t, max(0, B - 2 - int(m[r]))) for r in slots]
        rig.relay(slots, m, cand, bonus, suffix)
        anchors = bonus.astype(np.int32)
    log(f"relayed rows compared: {relayed_rows}")
    assert relayed_rows > 100
    rig.g.close()


def test_gpu_relay_with_conv():
    """The relay and the DFlash 2 two-tap convolution in the same drafts: the
    relayed rows enter the block as its inputs and the convolution then runs at
    all four sites of every layer (oracle: the convolution forward over the
    relayed block inputs).  Eight rounds of the relay workload."""
    from oracle import dflash2 as ds
    wl = synth.get_config("dflow_relay")
    d, bs, B = wl.dims, wl.bs, wl.dims.B
    rounds = 8
    log(f"case dflow relay + dflash2 conv: bs {bs}, B {B}, {rounds} rounds")
    rig = RelayRig(d, wl.seed, bs, max_ctx=wl.ctx[0] + rounds * B + B)
    cw = synth.make_conv_weights(d, wl.seed)
    rig.g.dr.conv_attach([{s: {k: rig.dfa.to_device(v) for k, v in t.items()} for s, t in layer.items()}
                          for layer in cw])
    cw32 = synth.conv_weights_as_f32(cw)
    slots = list(range(bs))
    rig.g.fuse(slots, wl.n_new, hidden_rows(d, wl.seed, [(r, 0, wl.n_new[r]) for r in range(bs)]))
    for r in range(bs):
        rig.o.fuse(r, synth.as_f32(synth.make_hidden(d, wl.seed, r, 0, wl.n_new[r])))
    anchors = synth.make_anchors(d, wl.seed, bs)
    nacc = synth.draw_accepted(bs, rounds, B, wl.seed)
    relayed = 0
    for t in range(rounds):
        ids, _, lg = rig.g.draft(slots, anchors, top_k=1, logits=True)
        cand = np.zeros((bs, B - 1), np.int32)
        for r in slots:
            relay_rows = rig.state.take(r)
            relayed += len(relay_rows)
            x0 = ofl.block_inputs(rig.w32, d, int(anchors[r]), relay_rows)
            ref = ds.draft_block_conv(rig.w32, d, rig.o.cache(r), int(anchors[r]), cw32, x0)["logits"]
            err = rel_inf(lg[r], ref)
            assert err <= 1e-4, f"round {t} req {r}: logits rel err {err}"
            _, bad = check_top1(ids[r][:, 0], ref)
            assert len(bad) == 0, f"round {t} req {r}: top-1 mismatch at {bad}"
            cand[r] = oracle.topk(ref, 1)[0][:, 0]
        m = nacc[t]
        tgt = synth.make_targets(cand, m, d.V, wl.seed * 1000 + t)
        tau, bonus = rig.g.accept(cand, 1, tgt)
        pos0 = [rig.o.cache(r).length for r in slots]
        rig.g.fuse(slots, [int(x) for x in tau], hidden_rows(d, wl.seed, [(r, pos0[r], int(tau[r])) for r in slots]))
        for r in slots:
            rig.o.fuse(r, synth.as_f32(synth.make_hidden(d, wl.seed, r, pos0[r], int(tau[r]))))
        suffix = [synth.make_suffix_hidden(d, wl.seed, r, t, max(0, B - 2 - int(m[r]))) for r in slots]
        rig.relay(slots, m, cand, bonus, suffix)
        anchors = bonus.astype(np.int32)
    log(f"relayed rows used: {relayed}")
    assert relayed > 10
    rig.g.close()


def test_gpu_relay_dropped_when_length_changes_or_reset():
    wl = synth.get_config("dflow_relay")
    d = wl.dims
    log("case dflow relay lifetime")
    rig = RelayRig(d, wl.seed, 2, max_ctx=256)
    rig.g.fuse([0, 1], [40, 40], hidden_rows(d, wl.seed, [(0, 0, 40), (1, 0, 40)]))
    cand = np.tile(np.arange(1, d.B, dtype=np.int32), (2, 1))
    suffix = [synth.make_suffix_hidden(d, wl.seed, r, 0, d.B - 2 - 3) for r in range(2)]
    rig.relay([0, 1], [3, 3], cand, np.array([5, 6], np.int32), suffix)
    assert rig.read_relay(0)[0] == d.B - 5 and rig.read_relay(1)[0] == d.B - 5
    rig.g.dr.slot_reset(0, 40)                 # rewind drops the relay
    assert rig.read_relay(0)[0] == 0
    rig.g.fuse([1], [1], hidden_rows(d, wl.seed, [(1, 40, 1)]))   # another length: stale
    assert rig.read_relay(1)[0] == 0
    # the draft then equals the plain draft
    o = oracle.OracleDrafter(rig.w32, d)
    o.fuse(1, synth.as_f32(synth.make_hidden(d, wl.seed, 1, 0, 41)))
    ids, _, lg = rig.g.draft([1], [7], top_k=1, logits=True)
    assert rel_inf(lg[0], o.draft(1, 7)["logits"]) <= 1e-4
    rig.g.close()


def test_gpu_relay_with_zero_second_layer_is_plain_draft():
    wl = synth.get_config("dflow_relay")
    d = wl.dims
    log("case dflow relay, w2 = 0")
    rig = RelayRig(d, wl.seed, 1, max_ctx=128)
    rig.rw_dev["w2"].zero_()
    rig.g.fuse([0], [30], hidden_rows(d, wl.seed, [(0, 0, 30)]))
    ids0, _, lg0 = rig.g.draft([0], [9], top_k=1, logits=True)
    cand = np.arange(1, d.B, dtype=np.int32)[None]
    rig.relay([0], [0], cand, np.array([9], np.int32), [synth.make_suffix_hidden(d, wl.seed, 0, 0, d.B - 2)])
    n, rows = rig.read_relay(0)
    assert n == d.B - 2
    assert np.array_equal(rows[2:2 + n], np.repeat(synth.as_f32([rig.w_np["e_mask"]])[0][None], n, 0))
    ids1, _, lg1 = rig.g.draft([0], [9], top_k=1, logits=True)
    assert np.array_equal(lg0, lg1) and np.array_equal(ids0, ids1)
    rig.g.close()


def test_gpu_relay_bf16_rows_qwen3_4b_shape():
    d = dataclasses.replace(QWEN3_4B, L=5)
    log("case dflow relay rows, Qwen3-4B shape bf16")
    rig = RelayRig(d, 9, 4, max_ctx=64)
    n_acc = [0, 5, 13, 15]
    cand = np.random.default_rng(0).integers(0, d.V, size=(4, d.B - 1)).astype(np.int32)
    bonus = np.array([11, 22, 33, 44], np.int32)
    suffix = [synth.make_suffix_hidden(d, 9, r, 0, max(0, d.B - 2 - n)) for r, n in enumerate(n_acc)]
    rig.relay([0, 1, 2, 3], n_acc, cand, bonus, suffix)
    for r in range(4):
        n, rows = rig.read_relay(r)
        want = rig.state.rows.get(r, {})
        assert n == len(want)
        for off, x in want.items():
            err = np.abs(rows[off] - x).max() / np.abs(x).max()
            assert err <= 2e-2, f"req {r} offset {off}: relay row err {err}"
    rig.g.close()
