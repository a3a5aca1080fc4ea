"""GPU parity of the gated delta rule (recurrent layers) against the oracle
(O8, token by token in double): chunked prefill with ragged tails, batches,
initial states, grouped key heads, weak and strong decay; the one-token decode
step; and the 32K-token layer in the benchmark's launch configuration on
sampled heads.

Tolerance of the chunked prefill. Its products take bf16 operands (unit
roundoff u = 2^-9) with fp32 accumulation: the state S and the chunk writes U
each time they enter a product, the per-chunk factors W, M and the inverse T
(as T diag(.)) once. Each rounding perturbs one product term by at most u
relative; summed over the terms of an output with random signs this stays a
few u relative to the size of the output, and the decay keeps it from
building up along the sequence (a CPU model with the same roundings gives
max |err| / max |o| = 0.3-0.5 % and mean |err| / rms(o) = 0.2-0.3 % for mean
decays from 0.93 to 0.99995, flat in sequence length). The bars leave a
margin of 4x: max |err| <= 2e-2 max |o| and mean |err| <= 1e-2 rms(o) per
(sequence, head); the final state max |err| <= 5e-2 rms(S) and mean |err| <=
1e-2 rms(S). A dropped term of the chunked form (the intra-chunk M U, a decay
factor, a write gate) moves outputs by tens of percent.

The decode step is the recurrence itself in fp32: state within 1e-5 relative
to its scale, output within one bf16 rounding.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gen.configs import GDN
from qsa_check import dev

pytestmark = pytest.mark.gpu

O_MAX_REL, O_MEAN_REL, S_MAX_REL, S_MEAN_REL = 2e-2, 1e-2, 5e-2, 1e-2


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_09_amd as q
    assert torch.cuda.is_available()
    return q


def f32dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def check_out(go, ref, what):
    err = np.abs(go - ref)
    scale_max = np.abs(ref).max()
    rms = np.sqrt((ref ** 2).mean())
    assert err.max() <= O_MAX_REL * scale_max, f"{what}: max err {err.max()} vs max|o| {scale_max}"
    assert err.mean() <= O_MEAN_REL * rms, f"{what}: mean err {err.mean()} vs rms {rms}"


def check_state(gs, ref, what):
    err = np.abs(gs - ref)
    rms = np.sqrt((ref ** 2).mean())
    assert err.max() <= S_MAX_REL * rms, f"{what}: state max err {err.max()} vs rms {rms}"
    assert err.mean() <= S_MEAN_REL * rms, f"{what}: state mean err {err.mean()} vs rms {rms}"


def run_prefill(qsa, q, k, v, g, beta, S0=None, scale=None, want_state=True):
    B, T, Hqk, dk = q.shape
    Hv = v.shape[2]
    desc = qsa.gdn_desc(Hqk, Hv, scale=scale)
    out = torch.empty((B, T, Hv, 128), dtype=torch.bfloat16, device="cuda")
    Sf = torch.empty((B, Hv, 128, 128), dtype=torch.float32, device="cuda") if want_state else None
    ws = qsa.workspace(qsa.qsa_gdn_prefill_workspace_size(desc, B, T))
    qsa.qsa_gdn_prefill(desc, dev(q), dev(k), dev(v), f32dev(g), f32dev(beta), out,
                        initial_state=None if S0 is None else f32dev(S0), final_state=Sf, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), (Sf.cpu().numpy().astype(np.float64) if want_state else None)


@pytest.mark.parametrize("B,T,Hqk,Hv,with_s0,shift", [
    (1, 700, 2, 4, False, 3.0),    # ragged tail: 10 chunks + 60 tokens
    (2, 333, 1, 2, True, 3.0),     # batch of two, carried initial states
    (1, 64, 4, 4, False, 3.0),     # exactly one chunk
    (1, 1, 1, 1, True, 3.0),       # one token
    (1, 1500, 2, 2, False, 8.0),   # long memory (mean decay 0.9997)
    (1, 200, 1, 3, True, 0.0),     # strong decay (mean 0.5), three value heads per key head
])
def test_gdn_prefill_matches_oracle(qsa, B, T, Hqk, Hv, with_s0, shift):
    seed = 900 + T + Hv
    print("[case] gdn prefill", B, T, Hqk, Hv, with_s0, shift, flush=True)
    q, k, v, g, beta = gen.gdn_inputs(seed, B, T, Hqk, Hv, decay_shift=shift)
    S0 = gen.gdn_state(seed, B, Hv) if with_s0 else None
    go, gs = run_prefill(qsa, q, k, v, g, beta, S0)
    for b in range(B):
        o_ref, s_ref = oracle.gdn(q[b], k[b], v[b], g[b], beta[b], S0=None if S0 is None else S0[b])
        for h in range(Hv):
            check_out(go[b, :, h], o_ref[:, h], f"b{b} h{h}")
            check_state(gs[b, h], s_ref[h], f"b{b} h{h}")


@pytest.mark.parametrize("B", [2, 4])
def test_gdn_prefill_many_heads_matches_oracle(qsa, B):
    # 32 value heads per sequence: with more (sequence, head) pairs the scan
    # gives each workgroup more value rows (two or four waves on a 256-CU
    # device), so these take the wider workgroup shapes; ragged tail, carried
    # states; the oracle runs a spread of heads
    T, Hqk, Hv = 150, 16, 32
    print("[case] gdn prefill many heads", B, T, Hqk, Hv, flush=True)
    q, k, v, g, beta = gen.gdn_inputs(77 + B, B, T, Hqk, Hv)
    S0 = gen.gdn_state(77 + B, B, Hv)
    go, gs = run_prefill(qsa, q, k, v, g, beta, S0)
    heads = [0, 1, 6, 15, 16, 23, 30, 31]
    for b in range(B):
        o_ref, s_ref = oracle.gdn(q[b], k[b], v[b], g[b], beta[b], S0=S0[b], heads=heads)
        for h in heads:
            check_out(go[b, :, h], o_ref[:, h], f"b{b} h{h}")
            check_state(gs[b, h], s_ref[h], f"b{b} h{h}")


def test_gdn_prefill_empty_sequence_passes_the_state_through(qsa):
    q, k, v, g, beta = gen.gdn_inputs(3, 2, 0, 1, 2)
    S0 = gen.gdn_state(3, 2, 2)
    _, gs = run_prefill(qsa, q, k, v, g, beta, S0)
    assert np.array_equal(gs, S0.astype(np.float64))
    _, gz = run_prefill(qsa, q, k, v, g, beta, None)
    assert not gz.any()


def test_gdn_prefill_in_place_state_and_split_sequence(qsa):
    # two calls carrying the state in place equal one call over the whole
    # sequence, within the prefill tolerance against the oracle
    T1, T2, Hqk, Hv = 300, 250, 2, 4
    q, k, v, g, beta = gen.gdn_inputs(31, 1, T1 + T2, Hqk, Hv)
    desc = qsa.gdn_desc(Hqk, Hv)
    S = torch.zeros((1, Hv, 128, 128), dtype=torch.float32, device="cuda")
    outs = []
    for a, e in ((0, T1), (T1, T1 + T2)):
        out = torch.empty((1, e - a, Hv, 128), dtype=torch.bfloat16, device="cuda")
        ws = qsa.workspace(qsa.qsa_gdn_prefill_workspace_size(desc, 1, e - a))
        qsa.qsa_gdn_prefill(desc, dev(q[:, a:e]), dev(k[:, a:e]), dev(v[:, a:e]), f32dev(g[:, a:e]),
                            f32dev(beta[:, a:e]), out, initial_state=S, final_state=S, workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    go = torch.cat(outs, 1).float().cpu().numpy().astype(np.float64)
    o_ref, s_ref = oracle.gdn(q[0], k[0], v[0], g[0], beta[0])
    for h in range(Hv):
        check_out(go[0, :, h], o_ref[:, h], f"h{h}")
        check_state(S.cpu().numpy()[0, h].astype(np.float64), s_ref[h], f"h{h}")


@pytest.mark.parametrize("B,Hqk,Hv", [(8, 2, 4), (3, 1, 3)])
def test_gdn_decode_matches_oracle(qsa, B, Hqk, Hv):
    print("[case] gdn decode", B, Hqk, Hv, flush=True)
    q, k, v, g, beta = gen.gdn_inputs(41 + B, B, 1, Hqk, Hv)
    S0 = gen.gdn_state(41 + B, B, Hv)
    desc = qsa.gdn_desc(Hqk, Hv)
    S = f32dev(S0)
    out = torch.empty((B, Hv, 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_gdn_decode(desc, dev(q[:, 0]), dev(k[:, 0]), dev(v[:, 0]), f32dev(g[:, 0]), f32dev(beta[:, 0]), S, out)
    torch.cuda.synchronize()
    go = out.float().cpu().numpy().astype(np.float64)
    gs = S.cpu().numpy().astype(np.float64)
    for b in range(B):
        o_ref, s_ref = oracle.gdn(q[b], k[b], v[b], g[b], beta[b], S0=S0[b])
        scale = np.abs(s_ref).max()
        assert np.abs(gs[b] - s_ref).max() <= 1e-5 * scale, f"b{b}"
        assert np.all(np.abs(go[b] - o_ref[0]) <= 2.0 ** -8 * np.abs(o_ref[0]) + 1e-6), f"b{b}"


def test_gdn_decode_steps_follow_the_recurrence(qsa):
    # 40 decode steps from a zero state against the oracle over the same tokens
    T, B, Hqk, Hv = 40, 2, 1, 2
    q, k, v, g, beta = gen.gdn_inputs(51, B, T, Hqk, Hv)
    desc = qsa.gdn_desc(Hqk, Hv)
    S = torch.zeros((B, Hv, 128, 128), dtype=torch.float32, device="cuda")
    out = torch.empty((B, T, Hv, 128), dtype=torch.bfloat16, device="cuda")
    for t in range(T):
        o_t = torch.empty((B, Hv, 128), dtype=torch.bfloat16, device="cuda")
        qsa.qsa_gdn_decode(desc, dev(q[:, t]), dev(k[:, t]), dev(v[:, t]), f32dev(g[:, t]), f32dev(beta[:, t]), S,
                           o_t)
        out[:, t] = o_t
    torch.cuda.synchronize()
    go = out.float().cpu().numpy().astype(np.float64)
    for b in range(B):
        o_ref, s_ref = oracle.gdn(q[b], k[b], v[b], g[b], beta[b])
        assert np.abs(S.cpu().numpy()[b] - s_ref).max() <= 1e-5 * np.abs(s_ref).max()
        assert np.all(np.abs(go[b] - o_ref) <= 2.0 ** -8 * np.abs(o_ref) + 1e-6)


def test_gdn_prefill_full_size_sampled_heads(qsa):
    # the 32K-token layer, one call as the benchmark times it; the oracle runs
    # the first and the last value head (they read different key heads)
    W = GDN["g1"]
    print("[case] gdn prefill full size", W.name, flush=True)
    q, k, v, g, beta = gen.gdn_inputs(W.seed, W.batch, W.T, W.Hqk, W.Hv)
    go, gs = run_prefill(qsa, q, k, v, g, beta, None)
    heads = [0, W.Hv - 1]
    o_ref, s_ref = oracle.gdn(q[0], k[0], v[0], g[0], beta[0], heads=heads)
    for h in heads:
        check_out(go[0, :, h], o_ref[:, h], f"h{h}")
        check_state(gs[0, h], s_ref[h], f"h{h}")
    assert np.isfinite(go).all()
