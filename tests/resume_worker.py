"""Worker of tests/test_resume_fresh_process.py, run in a fresh process.

usage: resume_worker.py {oracle|gpu} SEED T_ALL T0 T1 STATE_IN|- STATE_OUT O_OUT [--die]

Processes tokens [T0, T1) of the seeded T_ALL-token sequence (all 48 value heads on the
GPU, four on the oracle), resuming from STATE_IN (.npy, or '-' for zero),
writes the final state to STATE_OUT and the outputs to O_OUT (.npy), and with
--die kills itself with SIGKILL right after the files are on disk, as a job
that crashes after writing its checkpoint."""
import os
import signal
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

HEADS = [0, 5, 17, 47]


def main(argv):
    mode, seed, t_all, t0, t1, s_in, s_out, o_out = argv[:8]
    die = "--die" in argv
    seed, t_all, t0, t1 = int(seed), int(t_all), int(t0), int(t1)
    from inputs import synth
    inp = synth.gdr_inputs(seed, T=t_all)
    sl = slice(t0, t1)
    q, k, v, g, beta = (np.ascontiguousarray(x[:, sl]) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    s0 = None if s_in == "-" else np.load(s_in)
    if mode == "oracle":
        from oracle import gdr as ref
        o, s = ref.forward(q, k, v, g, beta, s0, heads=HEADS)
        o = o[:, :, HEADS]
    else:
        import torch
        import gated_delta_rule_amd as gdr_amd
        dev = torch.device("cuda:0")
        bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(dev)
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
        ot, st = gdr_amd.chunk_gated_delta_rule(bf(q), bf(k), bf(v), f32(g), f32(beta),
                                                None if s0 is None else f32(s0), output_final_state=True)
        torch.cuda.synchronize()
        o, s = ot.cpu().numpy(), st.cpu().numpy()
    for path, arr in ((s_out, s), (o_out, o)):
        with open(path, "wb") as f:
            np.save(f, arr)
            f.flush()
            os.fsync(f.fileno())
    if die:
        os.kill(os.getpid(), signal.SIGKILL)


if __name__ == "__main__":
    main(sys.argv[1:])
