"""The build's no-scratch check (CPU only): the parser of the compiler's
kernel resource-usage remarks finds kernels that spill and only those."""
from candidate_scoring_amd import build


def remarks(*kernels):
    lines = []
    for name, scratch in kernels:
        lines.append(f"cs_project.hip:10:1: remark: Function Name: {name} "
                     "[-Rpass-analysis=kernel-resource-usage]")
        lines.append("cs_project.hip:10:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]")
        lines.append(f"cs_project.hip:10:1: remark:     ScratchSize [bytes/lane]: {scratch} "
                     "[-Rpass-analysis=kernel-resource-usage]")
    return "\n".join(lines)


def test_no_spills_reported_for_clean_kernels():
    assert build.spilling_kernels(remarks(("k_a", 0), ("k_b", 0))) == []


def test_spilling_kernels_are_named_with_their_scratch():
    got = build.spilling_kernels(remarks(("k_a", 0), ("k_ring", 644), ("k_c", 0), ("k_d", 16)))
    assert got == [("k_ring", 644), ("k_d", 16)]


def test_scratch_line_without_a_kernel_name_is_ignored():
    text = "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 12 [-R]\n" + remarks(("k", 0))
    assert build.spilling_kernels(text) == []


def test_c_client_is_built_and_links():
    """The plain C caller used by the GPU tests is built and its libraries
    resolve (run without arguments it prints its usage and touches no GPU)."""
    import subprocess
    from pathlib import Path

    client = Path(__file__).resolve().parent / "c_client" / "cs_client"
    if not client.exists():
        import __graft_entry__
        import candidate_scoring_amd as cs
        from candidate_scoring_amd import build

        if not cs.LIBRARY.exists():
            build.build()
        __graft_entry__.build_c_client()
    r = subprocess.run([str(client)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage: cs_client IN OUT" in r.stderr, r.stderr
