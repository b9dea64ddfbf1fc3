"""Launch-shape tuning of libmpstep: variants built with other compile-time knobs, timed in
alternation on one resident workload.

The library's launch shape is fixed at compile time by the MPK_* macros of
csrc/internal.h (resident blocks per CU, XCD runs, chunks per norm block, ...).
This tool builds named variants with other values and times each pass of the
step -- the first and later accumulations, the norm (with the last micro-batch
folded in) and AdamW -- with HIP events, every variant once per round, so that
slow drifts of the machine fall on all of them alike.  Every variant gets its
own plan over the same buffers; the numbers are medians over rounds.

    python -m optimizer_step_tensor_amd.tune build NAME=FLAGS [NAME=FLAGS ...]
    python -m optimizer_step_tensor_amd.tune time WORKLOAD NAME[,NAME...] [--rounds R] [--reps N]
                                                   [--weights value|device]

`build` runs on any machine with hipcc (FLAGS: comma-separated -D options, or
empty for the defaults) and writes _build/tune/libmpstep_NAME.so; `time` needs
the GPU and those files.  A timing run prints one markdown table.  With
--weights device every pass reads its micro-batch weight from device memory,
as bench.py's step does; the default passes it as a launch argument.
"""
import argparse
import ctypes
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(ROOT, "_build", "tune")


def variant_path(name):
    return os.path.join(OUT, "libmpstep_%s.so" % name)


def cmd_build(specs):
    from . import build as B
    os.makedirs(OUT, exist_ok=True)
    for spec in specs:
        name, _, flags = spec.partition("=")
        extra = [f for f in flags.split(",") if f]
        B.build(out=variant_path(name), extra=extra)
        print("built", name, " ".join(extra) or "(defaults)", flush=True)


def cmd_time(workload, names, rounds, reps, weights_on="value"):
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import torch
    import inputs
    import optimizer_step_tensor_amd as mp
    from inputs import configs

    w = configs.make(workload)
    P, k = w.total, w.k
    dt16 = mp.MP_BF16 if w.dtype == inputs.BF16 else mp.MP_FP16
    model = mp.ModelState(w.numels, dt16, with_acc=True, layout="flat")
    for t, x in enumerate(model.master):
        inputs.fill_dev_f32(x, w.master_recipe(t))
    g16 = model.grad_buffers()
    for t, x in enumerate(g16):
        inputs.fill_dev_u16(x, w.grad_recipe(1, 0, t), w.dtype)
    weights = mp.mp_token_weights(w.token_counts(1))
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    hp = mp.adamw_hparams(**w.hp)
    cfg = mp.scaler_cfg(init_scale=1.0, enabled=False)
    on_dev = weights_on == "device"
    wdev = torch.tensor([weights[0], weights[-1]], dtype=torch.float32, device="cuda")
    whost = (ctypes.c_float * 2)(weights[0], weights[-1])
    base = wdev.data_ptr() if on_dev else ctypes.addressof(whost)
    wfirst, wlast = ctypes.c_void_p(base), ctypes.c_void_p(base + 4)
    libs = {}
    for n in names:
        L = mp._bind(ctypes.CDLL(variant_path(n)))
        N = len(w.numels)
        ne = (ctypes.c_int64 * N)(*w.numels)
        plan, gs, st = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        ptrs = [mp._ptrs(a) for a in (model.acc, model.master, model.m, model.v, model.w16)]
        assert L.mp_plan_create(N, ne, dt16, *ptrs, None, ctypes.byref(plan)) == 0
        assert L.mp_gradset_create(plan, mp._ptrs(g16), ctypes.byref(gs)) == 0
        assert L.mp_state_create(ctypes.byref(cfg), ctypes.byref(st)) == 0
        libs[n] = (L, plan, (ctypes.c_void_p * 1)(gs.value), st)
    passes = ("first", "accumulate", "norm", "adamw")
    res = {n: {p: [] for p in passes} for n in names}
    d = int(on_dev)
    for r in range(rounds + 1):                       # round 0 warms up
        for n in names:
            L, plan, gs, st = libs[n]
            for _ in range(reps):
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
                ev[0].record(stream)
                assert L.mp_accumulate_group(plan, gs, wfirst, 1, d, 1, sp) == 0
                ev[1].record(stream)
                assert L.mp_accumulate_group(plan, gs, wfirst, 1, d, 0, sp) == 0
                ev[2].record(stream)
                assert L.mp_unscale_check_norm_group(plan, st, gs, wlast, 1, d, 0,
                                                     ctypes.c_float(w.max_norm), sp) == 0
                ev[3].record(stream)
                assert L.mp_adamw_step_group(plan, st, gs, wlast, 1, d, 0, ctypes.byref(hp),
                                             sp) == 0
                ev[4].record(stream)
                assert L.mp_scaler_update(st, sp) == 0
                torch.cuda.synchronize()
                if r:
                    for i, p in enumerate(passes):
                        res[n][p].append(ev[i].elapsed_time(ev[i + 1]))
    bpp = {"first": 6, "accumulate": 10, "norm": 6, "adamw": 32}
    print("| variant | " + " | ".join("%s ms (GB/s)" % p for p in passes) + " | norm + AdamW, % of 8 TB/s |")
    print("|---" * (len(passes) + 2) + "|")
    for n in names:
        med = {p: statistics.median(res[n][p]) for p in passes}
        cells = ["%.4g (%.0f)" % (med[p], bpp[p] * P / med[p] / 1e6) for p in passes]
        fused = 38 * P / (med["norm"] + med["adamw"]) / 1e6 / 8000 * 100
        print("| %s | %s | %.1f |" % (n, " | ".join(cells), fused), flush=True)
    print("\n%s: %d parameters, medians of %d rounds x %d launches per pass, weights %s"
          % (workload, P, rounds, reps, "read on the device" if on_dev else "as launch arguments"))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    b = sub.add_parser("build")
    b.add_argument("specs", nargs="+", help="NAME=FLAGS, FLAGS a comma-separated list of -D options")
    t = sub.add_parser("time")
    t.add_argument("workload")
    t.add_argument("names")
    t.add_argument("--rounds", type=int, default=4)
    t.add_argument("--reps", type=int, default=2)
    t.add_argument("--weights", choices=("value", "device"), default="value")
    a = ap.parse_args()
    if a.cmd == "build":
        cmd_build(a.specs)
    else:
        cmd_time(a.workload, a.names.split(","), a.rounds, a.reps, a.weights)


if __name__ == "__main__":
    main()
