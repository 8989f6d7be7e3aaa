"""The library's calls from two host threads at once, each on its own stream.

The entry points keep no state between calls (no allocation, no caches, the
HIP error state is per thread), so two threads may drive the whole
routed-expert chain concurrently. Each thread runs the chain of the graph
test (gate_up GEMM + SwiGLU epilogue, the streaming SwiGLU forward and
backward, down GEMM + router multiply, combine, router multiply forward and
backward) several times on its own inputs and stream, starting together;
every iteration must equal a single-threaded run on the same inputs bit for
bit.
"""
import sys
import threading

import pytest
import torch

from tests.test_gpu_graph import Chain, assert_same

pytestmark = pytest.mark.gpu
ITERATIONS = 5


def say(msg):
    print(f"\n[gpu-threads] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.synchronize()


def test_two_threads_on_their_own_streams_match_a_single_thread():
    chains = [Chain(seed=71), Chain(seed=72)]
    want = []
    for c in chains:
        c.reset()
        c.step()
        torch.cuda.synchronize()
        want.append(c.snapshot())
    say("single-thread references taken")

    start = threading.Barrier(len(chains))
    errors = []

    def work(i):
        try:
            c = chains[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait(timeout=60)
                for it in range(ITERATIONS):
                    c.reset()
                    c.step()
                    got = c.snapshot()
                    s.synchronize()
                    assert_same(got, want[i], f"thread {i}, iteration {it}")
        except BaseException as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(chains))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    if errors:
        raise errors[0]
    say(f"{len(chains)} threads x {ITERATIONS} iterations equal the single-thread run")
