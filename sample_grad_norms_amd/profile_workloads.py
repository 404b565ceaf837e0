"""Runs one named workload a few times, for profiling with rocprofv3 (the
112-projection stack with independent inputs is profiled through bench.py).

    python sample_grad_norms_amd/profile_workloads.py NAME [--reps R] [--calib-copy]

NAME is one of:
  long_context_hutch  Hutchinson, B=1, T=32768, d=2048, p=8192, k=32
  long_context_exact  the exact explicit route on the same inputs
  hutchpp             Hutch++, B=4, T=4096, d=p=2048, budget 32
  single_layer        Hutchinson, B=8, T=1024, d=p=2048, k=32
  single_layer_gram   the exact Gram route on the same inputs
  shared_stack        the Llama-3.2-1B-shaped stack with q/k/v and gate/up
                      sharing their input (grouped Hutchinson, B=4, T=4096, k=32)
  sign_stack          the stack with +-1 projections stored as bits
  lora_routed         rank-16 LoRA factors of the stack, routed call (exact norms)
  dpsgd_step          DP-SGD-RC training steps on a random-init Llama-width stack
                      (2 decoder layers, B=4, T=2048, bf16): forward, backward 1,
                      the norm path, backward 2 of sum c_i l_i, noise, Adam
--calib-copy first runs one 1 GiB device-to-device copy, the reference the
counter summaries scale FETCH_SIZE and WRITE_SIZE by.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

NAMES = ("long_context_hutch", "long_context_exact", "hutchpp", "single_layer", "single_layer_gram", "shared_stack",
         "sign_stack", "lora_routed", "dpsgd_step")


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("name", choices=NAMES)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--calib-copy", action="store_true")
    a = ap.parse_args()
    import torch
    import sample_grad_norms_amd as dp
    import workloads
    dev = torch.device("cuda:0")
    if a.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    if a.name.startswith("long_context"):
        pr = workloads.config5(device=dev)
        fn = (lambda: dp.hutch(pr.A, pr.G, pr.P)) if a.name.endswith("hutch") else (lambda: dp.exact(pr.A, pr.G))
    elif a.name == "hutchpp":
        pr = workloads.config4(device=dev)
        fn = lambda: dp.hutchpp(pr.A, pr.G, pr.S, pr.P, k=pr.k)
    elif a.name == "shared_stack":
        layers = workloads.shared_input_stack(device=dev)
        fn = lambda: dp.hutch_grouped(layers, C_clip=1.0)
    elif a.name == "sign_stack":
        projs = [workloads.config3_projection(j, device=dev) for j in range(112)]
        gen = torch.Generator(device=dev)
        gen.manual_seed(2024)
        triples = [(q.A, q.G, dp.random_signs(q.G.shape[2], 32, device=dev, generator=gen)) for q in projs]
        fn = lambda: dp.hutch_sign_grouped(triples, 32, C_clip=1.0)
    elif a.name == "lora_routed":
        routed = [(A, G, None) for (A, G, _) in workloads.lora_stack(device=dev)]
        fn = lambda: dp.norms_routed(routed, 32)
    elif a.name == "dpsgd_step":
        from sample_grad_norms_amd.dpsgd_rc import RandomizedClipping
        from workloads import llama_block as lb
        shape = dict(layers=2, dim=2048, heads=32, kv_heads=8, hidden=8192, vocab=2048)
        model = lb.build(90, device=dev, dtype=torch.bfloat16, **shape)
        x, y = lb.batch(91, 4, 2048, shape["dim"], shape["vocab"], device=dev, dtype=torch.bfloat16)
        rc = RandomizedClipping(model, C=1.0, noise_multiplier=1.0, k=32)
        opt = torch.optim.Adam(rc.params, lr=1e-5)

        def fn():
            with rc.capture():
                losses = lb.per_sample_loss(model(x), y)
            n, c = rc.clip_factors(losses)
            rc.clipped_backward(losses, c)
            rc.add_noise()
            opt.step()
            opt.zero_grad(set_to_none=True)
    else:
        pr = workloads.config2(device=dev)
        fn = (lambda: dp.exact(pr.A, pr.G, route="gram")) if a.name.endswith("gram") else (lambda: dp.hutch(pr.A, pr.G, pr.P))
    for _ in range(a.reps):
        fn()
    torch.cuda.synchronize()
    print(f"{a.name}: {a.reps} calls done", flush=True)


if __name__ == "__main__":
    main()
