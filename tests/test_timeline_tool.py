"""The timeline tool's instrumentation finds every anchor in the verify kernels' source (so a
change to the kernel that moves a barrier is noticed on the CPU), and leaves the source
unchanged apart from the stamps."""

import os
import re

from gated_deltanet_speculative_amd import timeline

SRC = os.path.join(timeline.CSRC, "tree_verify.hip")


def test_instrumentation_inserts_every_stamp():
    src = open(SRC).read()
    out = timeline._instrument(src)
    stamps = re.findall(r"GDN_STAMP\((\d+)\);", out)
    # verify body: entry, first loads, six barriers, end; window body: entry, end
    assert sorted(int(k) for k in stamps) == sorted([0, 1, 2, 3, 4, 5, 6, 7, 10, 0, 10])
    assert out.count("GDN_STAMP_ARRIVAL(sreg);") == 1
    stripped = re.sub(r"^[ \t]*(GDN_R?STAMP\(\d+\);( GDN_R?STAMP\(\d+\);)?|GDN_STAMP_ARRIVAL\(sreg\);)\n", "", out,
                      flags=re.M)
    assert stripped.replace(timeline._STAMP_DEFS + "\n", "") == src
