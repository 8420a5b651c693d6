"""Host logic of the configuration search: candidate enumeration and the cache."""

import memory_bound_normalization_rmsnorm_amd as rn
from memory_bound_normalization_rmsnorm_amd import tune


def test_candidates_cover_the_row_and_include_the_default():
    default = rn.rmsnorm_select_config(16384, 4096, rn.BF16, 1, 1, 256, 2)
    cands = tune.candidates(16384, 4096, rn.BF16, 1, 256, default)
    assert tune._key(cands[0]) == tune._key(default)
    nvec = 4096 * 2 // 16
    shapes = set()
    for c in cands:
        assert c.lanes_per_row * c.vecs_per_lane >= nvec
        assert (c.vecs_per_lane - 1) * c.lanes_per_row < nvec      # at most one partial slot
        assert c.wg_threads % c.lanes_per_row == 0
        assert 1 <= c.grid <= -(-16384 // (c.wg_threads // c.lanes_per_row))
        shapes.add((c.lanes_per_row, c.vecs_per_lane))
    assert {(64, 8), (128, 4), (256, 2), (512, 1)} <= shapes
    assert (1024, 1) not in shapes                                 # half of its lanes would be idle


def test_candidates_for_widths_the_vector_path_cannot_take():
    default = rn.rmsnorm_select_config(10, 70001, rn.F32, 0, 1, 256, 2)     # wider than the element kernels
    assert [tune._key(c) for c in tune.candidates(10, 70001, rn.F32, 0, 256, default)] == [tune._key(default)]
    # up to 16384 columns: element kernels, the widest group N allows and single elements, every row size
    # that holds the row in 16 elements per lane
    for M, N, dt, g in ((4096, 4100, rn.BF16, 4), (4096, 4098, rn.F32, 2), (4096, 4100, rn.BF16_WF32, 4),
                        (100, 4095, rn.F16, 1), (3000, 13, rn.F32, 1)):
        for d in (0, 1):
            default = rn.rmsnorm_select_config(M, N, dt, d, 1, 256, 2)
            cands = tune.candidates(M, N, dt, d, 256, default)
            assert tune._key(cands[0]) == tune._key(default)
            assert (default.vector_path, default.elems_per_access) == (3, g)
            want = {(gg, lanes, -(-N // (lanes * gg))) for gg in {g, 1} for lanes in (64, 128, 256, 512, 1024)
                    if -(-N // (lanes * gg)) * gg <= 16}
            assert {(c.elems_per_access, c.lanes_per_row, c.vecs_per_lane) for c in cands[1:]} == want
            grids = {c.grid for c in cands[1:]}
            assert max(grids) == M and (256 in grids or M < 256) and all(1 <= x <= M for x in grids)
            for c in cands[1:]:
                assert (c.vector_path, c.wg_threads, c.prefetch) == (3, c.lanes_per_row, 0)


def test_cache_round_trip(tmp_path):
    cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=128, vecs_per_lane=4, wg_threads=512, prefetch=1, grid=77)
    path = str(tmp_path / "sub" / "tuned.json")
    key = tune.cache_key(16384, 4096, rn.BF16, 0, "dev", 256)
    assert "fwd" in key and "16384" in key and rn.rmsnorm_build_info() in key
    tune.save_cache(path, {key: {"config": cfg.as_dict()}})
    back = tune.config_from_dict(tune.load_cache(path)[key]["config"])
    assert tune._key(back) == tune._key(cfg)
    assert tune.load_cache(str(tmp_path / "missing.json")) == {}


def test_candidates_include_whole_wavefront_backward_rows():
    """Backward rows of 257-1023 vectors whose whole wavefronts are not a power
    of two: the workgroup-sized row kernels, at both prefetch depths."""
    cands = tune.candidates(16384, 5120, rn.BF16, 1, 256)
    rowwg = {(c.lanes_per_row, c.wg_threads, c.prefetch) for c in cands if c.lanes_per_row == 640 and not c.copy_mode}
    assert rowwg == {(640, 640, 1), (640, 640, 2)}


def test_candidates_include_the_lds_pipeline():
    """The backward's memory path is a search dimension: LDS-staged
    configurations (copy_mode 1) at every built stage count, for power-of-two
    rows and for rows on whole wavefronts, at one and two workgroups per CU;
    none for the forward or for rows of more than one vector per lane."""
    def lds(M, N, dt=rn.BF16, is_bwd=1):
        return {(c.lanes_per_row, c.wg_threads, c.prefetch, c.grid)
                for c in tune.candidates(M, N, dt, is_bwd, 256) if c.copy_mode == 1 and c.vector_path == 1}
    assert lds(16384, 4096) == {(512, 512, s, g) for s in (2, 3, 4, 6, 8) for g in (256, 512)}
    assert {(l, s) for l, _, s, _ in lds(16384, 5120)} == {(l, s) for l in (640, 1024) for s in (2, 3, 4)}
    assert {(l, w) for l, w, _, _ in lds(16384, 2048)} == {(256, 1024)}
    assert lds(16384, 4096, is_bwd=0) == set()
    assert lds(4096, 32768) == set()           # 4096 vectors: the wide-row kernels (below)
    wide = {(c.lanes_per_row, c.vecs_per_lane, c.prefetch) for c in tune.candidates(4096, 32768, rn.BF16, 1, 256)
            if c.copy_mode == 1 and c.vector_path == 2}
    assert wide == set()                       # 32768 columns: none built (they spill)
    wide = {(c.lanes_per_row, c.vecs_per_lane, c.prefetch) for c in tune.candidates(4096, 16384, rn.F16, 1, 256)
            if c.copy_mode == 1 and c.vector_path == 2}
    assert wide == {(1024, 2, 1), (1024, 2, 2), (512, 4, 1), (512, 4, 2)}
    assert not any(c.copy_mode for c in tune.candidates(4096, 32768, rn.F32, 1, 256))
    assert lds(4096, 1024) == set()            # 128 vectors
    assert not [c for c in tune.candidates(16384, 5120, rn.BF16, 0, 256) if c.lanes_per_row == 640]  # forward
    assert not [c for c in tune.candidates(16384, 4096, rn.BF16, 1, 256) if c.lanes_per_row % 64 == 0 and
                c.lanes_per_row & (c.lanes_per_row - 1)]                                           # 512: a power of two


def test_candidates_include_split_rows_and_the_widest_forward():
    """Backward rows beyond the wide kernels: the split-row kernels at the
    fewest members and one more, every built prefetch, whole resident groups;
    forward rows of 9 to 16 vectors per lane on 1024 lanes."""
    M, N = 4096, 98304  # bf16: 12288 vectors: 3 or 4 members of 4 or 3 per lane, 6 or 7 of 2
    default = rn.rmsnorm_select_config(M, N, rn.BF16, 1, 1, 256, 2)
    cands = tune.candidates(M, N, rn.BF16, 1, 256, default)
    split = {(c.lanes_per_row // 1024, c.vecs_per_lane, c.prefetch, c.grid) for c in cands if c.vector_path == 4}
    assert split == {(3, 4, 0, 255), (3, 4, 1, 255), (3, 4, 0, 129), (3, 4, 1, 129),
                     (4, 3, 0, 256), (4, 3, 1, 256), (4, 3, 0, 128), (4, 3, 1, 128),
                     (6, 2, 0, 510), (6, 2, 0, 258), (7, 2, 0, 511), (7, 2, 0, 259)}
    assert tune._key(cands[0]) == tune._key(default) and default.vector_path == 4
    # fp32 weights: no prefetch variant; fp32 activations: 5 to 8 vectors per lane
    assert {c.prefetch for c in tune.candidates(M, N, rn.BF16_WF32, 1, 256) if c.vector_path == 4} == {0}
    assert {(c.lanes_per_row // 1024, c.vecs_per_lane) for c in tune.candidates(M, 40960, rn.F32, 1, 256)
            if c.vector_path == 4} == {(2, 5)}
    fwd = [c for c in tune.candidates(M, 131072, rn.BF16, 0, 256) if c.vector_path == 1 and c.vecs_per_lane > 8]
    assert fwd and all((c.vector_path, c.lanes_per_row, c.vecs_per_lane, c.wg_threads) == (1, 1024, 16, 1024)
                       for c in fwd)
    # the two-pass forward: every built (chunk, kept, LDS) shape, a workgroup per row or two per CU
    loop = {(c.vecs_per_lane, c.kept_vecs, c.copy_mode, c.grid) for c in tune.candidates(M, 262144, rn.BF16, 0, 256)
            if c.vector_path == 5}
    assert loop == {(ch, kv, l, g) for ch, kv, l in ((4, 0, 0), (8, 0, 0), (16, 0, 0), (4, 16, 0), (4, 12, 0),
                                                     (2, 16, 1), (4, 16, 1), (4, 12, 1)) for g in (4096, 512)}
    assert {(c.vecs_per_lane, c.kept_vecs, c.copy_mode) for c in tune.candidates(M, 262144, rn.BF16_WF32, 0, 256)
            if c.vector_path == 5} == {(4, 0, 0), (8, 0, 0), (2, 14, 0), (2, 10, 1)}
