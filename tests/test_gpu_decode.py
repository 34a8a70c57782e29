"""GPU parity of attn_decode (split + combine) against the fp64 oracle.

Small cases run the oracle on every output; the full-size workloads compare a
sample of (sequence, head) outputs that the oracle computes one by one, with
the same launch configuration the benchmark times.
"""

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_gqa_amd import binding, inputs
import parity_utils as pu

pytestmark = pytest.mark.gpu

DEV = "cuda"


def wl(name, B, h_q, n_kv, d, S, qd, kd, lens=None, seed=100):
    lens = lens or (S, S)
    return inputs.DecodeWorkload(name, B=B, h_q=h_q, n_kv=n_kv, d_h=d, S_max=S, q_dtype=qd, kv_dtype=kd,
                                 lens=lens, seed=seed)


def check_full(inp, n_split=0, tol=None):
    print(f"[decode] {inp.wl} lens={inp.seq_lens.tolist()} n_split={n_split}", flush=True)
    out = pu.run_decode(inp, n_split=n_split)
    pu.sync()
    ref = pu.oracle_decode_full(inp)
    err = pu.max_err(out, ref)
    tol = tol or pu.TOL[inp.wl.kv_dtype]
    assert err <= tol, f"max abs err {err} > {tol}"
    return out, err


# ------------------------------------------------------------- the workloads

def test_mqa_tiny_f32_full():
    inp = inputs.make_decode_inputs(inputs.MQA_TINY_F32, device=DEV)
    check_full(inp)


@pytest.mark.parametrize("name", ["gqa_decode_ragged_bf16", "mqa_decode_long_bf16", "gqa_decode_fp8kv",
                                  "gqa_decode_int8kv", "gqa_decode_int4kv"])
def test_full_size_workload_every_row(name):
    """The benchmarked workloads at full size in the benchmark's launch
    configuration: every (sequence, head) output row against the oracle,
    which decodes one (sequence, kv-head) slab at a time."""
    w = {**inputs.DECODE_WORKLOADS, **inputs.QUANT_DECODE_WORKLOADS}[name]
    inp = inputs.make_decode_inputs(w, device=DEV)
    print(f"[decode-full] {name} sumL={int(inp.seq_lens.sum())}", flush=True)
    out = pu.run_decode(inp)
    pu.sync()
    ref = pu.oracle_decode_every_row(
        inp, progress=lambda b: print(f"[decode-full] {name} oracle b={b}", flush=True) if b % 8 == 7 else None)
    err = pu.max_err(out, ref)
    print(f"[decode-full] {name} max abs err {err:.3e} over {w.B * w.h_q} rows", flush=True)
    assert err <= pu.TOL[w.kv_dtype], f"{name}: max abs err {err}"


# ------------------------------------------------------ reduced, all outputs

@pytest.mark.parametrize("kd", ["bf16", "fp8", "int8", "int4"])
def test_gqa_ragged_poisoned_tails(kd):
    w = wl("ragged", B=5, h_q=64, n_kv=8, d=128, S=520, qd="bf16", kd=kd, seed=7)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[1, 33, 300, 520, 97], poison_tail=True)
    check_full(inp)


def test_mqa_long_ragged_tile_tail():
    w = wl("mqa", B=3, h_q=32, n_kv=1, d=128, S=1000, qd="bf16", kd="bf16", seed=8)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[1000, 999, 64], poison_tail=True)
    check_full(inp)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8", "int8", "int4"])
@pytest.mark.parametrize("d", [64, 128])
def test_group_size_sweep(G, kd, d):
    n_kv = 2 if G <= 32 else 1
    qd = "f32" if kd == "f32" else "bf16"
    w = wl("sweep", B=2, h_q=G * n_kv, n_kv=n_kv, d=d, S=200, qd=qd, kd=kd, seed=G * 10 + d)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[200, 77], poison_tail=True)
    check_full(inp)


@pytest.mark.parametrize("n_split", [1, 2, 7, 10 ** 6])
@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8", "int8", "int4"])
def test_forced_splits_agree(n_split, kd):
    qd = "f32" if kd == "f32" else "bf16"
    w = wl("splits", B=3, h_q=16, n_kv=2, d=128, S=700, qd=qd, kd=kd, seed=31)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[700, 450, 1], poison_tail=True)
    desc = binding.decode_desc(inp.q, inp.k, n_split)
    print(f"[decode] effective n_split={binding.attn_decode_num_splits(desc)}", flush=True)
    check_full(inp, n_split=n_split)


@pytest.mark.parametrize("n_split", [0, 3, 10 ** 6])
def test_int4_tile_halves(n_split):
    """int4 with one block of 16 heads schedules 64-token tiles held as two
    32-token register halves: lengths on both sides of every half boundary
    (the second half empty, partly or wholly filled), with the key ranges
    cut at the library's count, at 3, and at every tile."""
    lens = [31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129]
    w = wl("int4-halves", B=len(lens), h_q=16, n_kv=2, d=128, S=160, qd="bf16", kd="int4", seed=49)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=lens, poison_tail=True)
    check_full(inp, n_split=n_split)


@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8", "int4"])
def test_more_than_64_sequences(kd):
    """B > 64: the split and combine kernels find the slabs by scanning the
    lengths 64 at a time instead of one lane per sequence."""
    qd = "f32" if kd == "f32" else "bf16"
    w = wl("wide", B=70, h_q=16, n_kv=2, d=64, S=160, qd=qd, kd=kd, lens=(0, 160), seed=51)
    check_full(inputs.make_decode_inputs(w, device=DEV, poison_tail=True))


@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8", "int8", "int4"])
def test_empty_and_overlong_lengths(kd):
    qd = "f32" if kd == "f32" else "bf16"
    w = wl("edge", B=4, h_q=8, n_kv=2, d=128, S=96, qd=qd, kd=kd, seed=41)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[0, 96, 5000, -3])
    out, _ = check_full(inp)
    assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[3]) == 0


def test_single_key_returns_value_row():
    w = wl("one", B=2, h_q=8, n_kv=2, d=128, S=64, qd="bf16", kd="bf16", seed=43)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[1, 1])
    out = pu.run_decode(inp)
    pu.sync()
    for j in range(8):
        assert torch.equal(out[:, j], inp.v[:, j // 4, 0])  # p = 1 exactly; bf16 value passes through


@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8", "int8", "int4"])
@pytest.mark.parametrize("h_q", [16, 64])
def test_zero_scale_gives_the_mean_of_visible_values(kd, h_q):
    """scale = 0: every visible key has the same weight, so each output row is
    the mean of the sequence's visible V rows (the oracle at scale 0)."""
    qd = "f32" if kd == "f32" else "bf16"
    w = wl("zero", B=3, h_q=h_q, n_kv=2, d=128, S=300, qd=qd, kd=kd, seed=61)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[1, 300, 77])
    out = binding.attn_decode(inp.q, inp.k, inp.v, inp.seq_lens, 0.0, k_scale=inp.k_scale, v_scale=inp.v_scale)
    pu.sync()
    q = pu.to_f64(inp.q)
    lens = inp.seq_lens.cpu().tolist()
    ref = np.zeros(tuple(out.shape))
    for b in range(w.B):
        for g in range(w.n_kv):
            k, v = pu.cache_f64(inp, b, g)
            for j in range(g * w.G, (g + 1) * w.G):
                ref[b, j] = oracle.attend_one_row(q[b, j], k[:lens[b]], v[:lens[b]], 0.0)
    assert pu.max_err(out, ref) <= pu.TOL[kd]


@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8", "int8", "int4"])
def test_deterministic_repeat(kd):
    """Repeated calls agree bitwise where the summation order is fixed: always
    on the float32 path, and on the matrix-core paths when each wave reduces at
    most one tile of its workgroup's range (true at this size: at most 5 tiles
    per range, 8 waves)."""
    qd = "f32" if kd == "f32" else "bf16"
    w = wl("det", B=4, h_q=32, n_kv=4, d=128, S=2048, qd=qd, kd=kd, lens=(100, 2048), seed=47)
    inp = inputs.make_decode_inputs(w, device=DEV)
    a = pu.run_decode(inp).clone()
    b = pu.run_decode(inp)
    pu.sync()
    assert torch.equal(a, b)


@pytest.mark.parametrize("kd", ["bf16", "fp8", "int8", "int4"])
def test_repeat_at_full_size_deterministic_is_bitwise(kd):
    """With GQA_DECODE_DETERMINISTIC every wave keeps a fixed tile order, so
    two identical full-size calls give the same bits (the exact method has one
    result; this pins that the kernel's rounding does not depend on timing)."""
    w = {"bf16": inputs.GQA_RAGGED_BF16, "fp8": inputs.GQA_FP8KV, "int8": inputs.GQA_INT8KV,
         "int4": inputs.GQA_INT4KV}[kd]
    inp = inputs.make_decode_inputs(w, device=DEV)
    a = binding.attn_decode(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, k_scale=inp.k_scale, v_scale=inp.v_scale,
                            deterministic=True).clone()
    for _ in range(2):
        b = binding.attn_decode(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, k_scale=inp.k_scale,
                                v_scale=inp.v_scale, deterministic=True)
        pu.sync()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_repeat_at_full_size_mqa_deterministic_is_bitwise():
    w = inputs.MQA_LONG_BF16
    inp = inputs.make_decode_inputs(w, device=DEV)
    a = binding.attn_decode(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, deterministic=True).clone()
    b = binding.attn_decode(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, deterministic=True)
    pu.sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("n_split", [0, 3, 10 ** 6])
@pytest.mark.parametrize("kd", ["bf16", "fp8", "int8", "int4"])
def test_deterministic_mode_matches_oracle(kd, n_split):
    """The deterministic tile order gives the same exact result (within the
    bar) for several tiles per wave, segment boundaries and split counts."""
    w = wl("det-oracle", B=5, h_q=64, n_kv=4, d=128, S=3000, qd="bf16", kd=kd, seed=57)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[3000, 1, 1777, 640, 2999], poison_tail=True)
    out = binding.attn_decode(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, k_scale=inp.k_scale, v_scale=inp.v_scale,
                              n_split=n_split, deterministic=True)
    pu.sync()
    err = pu.max_err(out, pu.oracle_decode_full(inp))
    assert err <= pu.TOL[kd], f"max abs err {err}"


def test_default_split_count_is_the_device_cu_count():
    """n_split = 0 takes one workgroup per compute unit of the current device."""
    w = inputs.GQA_RAGGED_BF16
    q = torch.empty((w.B, w.h_q, w.d_h), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((w.B, w.n_kv, w.S_max, w.d_h), dtype=torch.bfloat16, device=DEV)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert binding.attn_decode_num_splits(binding.decode_desc(q, k)) == cus


@pytest.mark.parametrize("kd", ["bf16", "fp8", "int8", "int4"])
def test_repeat_at_full_size(kd):
    """With several tiles per wave the waves take tiles as they free up, so two
    identical calls may differ in float32 summation order and in where each
    wave rounds its probabilities to bf16: the outputs stay within about 1e-3
    of each other (4e-3 allowed), far inside the accuracy bar."""
    w = {"bf16": inputs.GQA_RAGGED_BF16, "fp8": inputs.GQA_FP8KV, "int8": inputs.GQA_INT8KV,
         "int4": inputs.GQA_INT4KV}[kd]
    inp = inputs.make_decode_inputs(w, device=DEV)
    a = pu.run_decode(inp).clone()
    b = pu.run_decode(inp)
    pu.sync()
    assert (a.float() - b.float()).abs().max().item() <= 4e-3


def test_partials_then_combine_equals_decode():
    w = wl("halves", B=4, h_q=64, n_kv=8, d=128, S=1500, qd="bf16", kd="bf16", lens=(1, 1500), seed=53)
    inp = inputs.make_decode_inputs(w, device=DEV)
    full = pu.run_decode(inp)
    desc = binding.decode_desc(inp.q, inp.k)
    ws = torch.empty(binding.attn_decode_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    binding.attn_decode_partials(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, ws)
    out = torch.empty_like(inp.q)
    binding.attn_decode_combine(inp.q, inp.k, inp.seq_lens, ws, out)
    pu.sync()
    assert torch.equal(out, full)


@pytest.mark.parametrize("kd", ["bf16", "fp8", "int8", "int4"])
def test_workspace_reused_across_calls(kd):
    """One workspace, filled with NaN bit patterns once, serves calls with
    different lengths and split counts; every result matches the oracle."""
    w = wl("reuse", B=6, h_q=32, n_kv=4, d=128, S=900, qd="bf16", kd=kd, seed=61)
    base = inputs.make_decode_inputs(w, device=DEV)
    cases = [([900, 1, 450, 0, 33, 899], 0), ([5, 5, 5, 5, 5, 5], 0), ([900] * 6, 3), ([1, 64, 2, 0, 700, 31], 10 ** 6),
             ([0] * 6, 0), ([321, 654, 87, 900, 12, 1], 17)]
    need = max(binding.attn_decode_workspace_bytes(binding.decode_desc(base.q, base.k, ns)) for _, ns in cases)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    for lens, ns in cases:
        inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=lens, poison_tail=True)
        print(f"[decode-reuse] {kd} lens={lens} n_split={ns}", flush=True)
        out = torch.full_like(inp.q, float("nan"))
        pu.run_decode(inp, n_split=ns, out=out, workspace=ws)
        pu.sync()
        err = pu.max_err(out, pu.oracle_decode_full(inp))
        assert err <= pu.TOL[kd], f"lens={lens} n_split={ns}: max abs err {err}"


def test_all_sequences_empty_gives_zero_rows():
    w = wl("allempty", B=3, h_q=16, n_kv=2, d=64, S=128, qd="bf16", kd="bf16", seed=67)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[0, 0, 0])
    out = torch.full_like(inp.q, float("nan"))
    pu.run_decode(inp, out=out)
    pu.sync()
    assert torch.count_nonzero(out) == 0


@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8", "int8", "int4"])
def test_prepared_call_matches_plain_call(kd):
    qd = "f32" if kd == "f32" else "bf16"
    w = wl("prep", B=3, h_q=16, n_kv=2, d=128, S=300, qd=qd, kd=kd, seed=71)
    inp = inputs.make_decode_inputs(w, device=DEV, seq_lens=[300, 2, 150])
    ref = pu.run_decode(inp)
    desc = binding.decode_desc(inp.q, inp.k)
    ws = torch.empty(binding.attn_decode_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(inp.q)
    call = binding.prepare_decode(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, out, ws, k_scale=inp.k_scale,
                                  v_scale=inp.v_scale)
    for _ in range(3):
        out.fill_(float("nan"))
        assert call() is out
        pu.sync()
        assert torch.equal(out, ref)


def test_temporary_workspace_lives_on_the_call_stream():
    """With no workspace given, the call allocates one on the stream its
    kernels run on.  The side stream is first held back by a long matrix
    product; the default stream then allocates and fills tensors of the
    workspace's size at once.  Had the workspace come from the default
    stream's pool, those fills could overwrite the partials before the
    combine kernel reads them."""
    w = wl("ws-stream", B=4, h_q=64, n_kv=8, d=128, S=2048, qd="bf16", kd="bf16", lens=(1024, 2048), seed=63)
    inp = inputs.make_decode_inputs(w, device=DEV)
    ref = pu.run_decode(inp).clone()
    need = binding.attn_decode_workspace_bytes(binding.decode_desc(inp.q, inp.k))
    a = torch.randn(4096, 4096, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = torch.empty_like(inp.q)
    with torch.cuda.stream(s):
        for _ in range(20):
            a = a @ a * 1e-3  # keeps the side stream busy for a while
    binding.attn_decode(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, out=out, stream=s)
    junk = [torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV) for _ in range(4)]
    s.synchronize()
    pu.sync()
    del junk
    assert torch.equal(out, ref)


def test_runs_on_a_side_stream():
    w = wl("stream", B=2, h_q=16, n_kv=2, d=128, S=512, qd="bf16", kd="bf16", seed=59)
    inp = inputs.make_decode_inputs(w, device=DEV)
    ref = pu.run_decode(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = pu.run_decode(inp)
    s.synchronize()
    pu.sync()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 * (1 << 20) + 48, 1 << 28])
def test_stream_read_runs_and_writes_nothing_else(nbytes):
    """The read-only stream (the measured HBM ceiling) reads any multiple of
    16 bytes, leaves the buffer unchanged and touches nothing but its sink."""
    buf = torch.arange(nbytes // 4, dtype=torch.int32, device=DEV)
    before = buf.clone()
    sink = torch.zeros(2, dtype=torch.int32, device=DEV)
    binding.gqa_stream_read(buf, sink[:1])
    pu.sync()
    assert torch.equal(buf, before)
    assert int(sink[1]) == 0
