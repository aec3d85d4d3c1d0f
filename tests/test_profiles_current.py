"""Every committed rocprofv3 summary under profiles/ names the command that
made it (running committed files only) and the hash of the kernel sources it
was taken on, and that hash is the current one: a summary left over from
changed kernels would describe launches that no longer exist."""
import hashlib
import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
GDN_SRC = os.path.join(ROOT, "skinny_bit_block_amd", "csrc", "gdn_kernels.hip")


def profile_files():
    return sorted(f for f in os.listdir(PROFILES) if f.endswith((".md", ".txt")))


def test_profiles_are_text_summaries():
    files = profile_files()
    assert files
    assert set(os.listdir(PROFILES)) == set(files)  # nothing but the summaries
    for f in files:
        assert os.path.getsize(os.path.join(PROFILES, f)) < 64 * 1024, f


def test_profiles_name_their_command_and_current_source():
    qmm_sha = bench.kernel_source_sha()
    gdn_sha = hashlib.sha256(open(GDN_SRC, "rb").read()).hexdigest()[:16]
    for f in profile_files():
        text = open(os.path.join(PROFILES, f)).read()
        assert "rocprofv3" in text, f  # the command that made it
        m = re.search(r"^kernel_source_sha256:\s*(.+)$", text, re.M)
        assert m, f
        sha = m.group(1).strip()
        if f.startswith("gdn_"):
            assert sha == "gdn_kernels.hip %s" % gdn_sha, f
        else:
            assert sha == qmm_sha, f
        # commands run committed files only (no scratch paths)
        assert "_work" not in text, f
