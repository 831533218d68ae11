"""Run every oracle pin against one build of the oracle (path in argv[1]).

Exit status: 0 with "CAUGHT <check>" printed when a pin fails, 3 when every
pin passes. Used by the mutation tests in a child process.
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import oracle_pins as P  # noqa: E402

if __name__ == "__main__":
    with oracle.using(sys.argv[1]):
        for check in P.ALL:
            try:
                check()
            except AssertionError as e:
                print("CAUGHT", check.__name__, str(e)[:120], flush=True)
                sys.exit(0)
    print("NOT CAUGHT", flush=True)
    sys.exit(3)
