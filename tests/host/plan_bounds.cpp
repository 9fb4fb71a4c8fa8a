// Host bounds harness of the selective-scan library's plans (ss_plan.h), built with
// -fsanitize=address,undefined by tests/test_sanitize.py.
//
// For every dims it tries (the benchmark workloads, shapes past 2^31 elements, a seeded sweep
// of the option space, and invalid or overflowing dims) it checks that each workspace region
// the plan carves is 256-byte aligned, lies inside [0, ws_total) and overlaps no other region,
// with every region's size recomputed here from the dims in 128-bit arithmetic.  Invalid dims
// must come back as errors; the sanitizers catch any overflow or out-of-range access on the
// way.  Prints "plan bounds ok <count>" and exits 0, or names the first failing case.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "ss_plan.h"

namespace {

using u128 = unsigned __int128;

struct Region {
    const char* name;
    size_t off;
    u128 bytes;
};

int g_cases = 0;

void fail(const char* what, const ss_dims& d, int backward) {
    std::printf("FAIL %s: B=%" PRId64 " L=%" PRId64 " D=%" PRId64 " N=%" PRId64
                " dtype=%d plan=%d chunk=%" PRId64 " layout=%d disc=%d order=%d dt=%d bwd=%d\n",
                what, d.batch, d.seqlen, d.dim, d.dstate, d.in_dtype, d.plan, d.chunk, d.layout,
                d.disc, d.order, d.dt_layout, backward);
    std::exit(1);
}

void check_regions(const std::vector<Region>& rs, u128 total, const ss_dims& d, int bwd) {
    for (size_t i = 0; i < rs.size(); ++i) {
        if (rs[i].off % 256 != 0) fail(rs[i].name, d, bwd);
        if (u128(rs[i].off) + rs[i].bytes > total) fail(rs[i].name, d, bwd);
        for (size_t j = 0; j < i; ++j) {
            const u128 a0 = rs[i].off, a1 = a0 + rs[i].bytes, b0 = rs[j].off, b1 = b0 + rs[j].bytes;
            if (rs[i].bytes && rs[j].bytes && a0 < b1 && b0 < a1) fail("overlap", d, bwd);
        }
    }
}

void check_scan(const ss_dims& d) {
    for (int bwd = 0; bwd < 2; ++bwd) {
        ss::Plan p;
        const int rc = ss::make_plan(d, bwd ? ss::kPlanBwd : ss::kPlanFwd, &p);
        ++g_cases;
        if (rc != SS_OK) continue;
        const u128 B = u128(p.B), L = u128(p.L), D = u128(p.D), N = u128(p.N), K = u128(p.K);
        if (K * u128(p.chunk) < L || (K - 1) * u128(p.chunk) >= L) fail("chunk count", d, bwd);
        std::vector<Region> rs;
        if (!bwd && !p.group) rs.push_back({"bc staging", p.off_bc, B * L * 2 * N * 4});
        if (p.chunked) {
            rs.push_back({"h_end", p.off_hend, B * K * D * N * 4});
            rs.push_back({"dsum", p.off_dsum, B * K * D * 4});
            if (bwd) {
                const u128 NB = (D + 63) / 64;
                if (u128(ss::bwd_reduce_blocks(p)) != NB) fail("channel blocks", d, bwd);
                rs.push_back({"reverse pairs", p.off_gend, B * K * D * N * 4});
                rs.push_back({"dB|dC partials", p.off_bcpart, B * NB * L * 2 * N * 4});
                rs.push_back({"dD|ddt_bias partials", p.off_dtpart, B * K * D * 2 * 4});
                if (p.dt_shared) rs.push_back({"shared dt partials", p.off_ddt, B * NB * L * 4});
            } else {
                rs.push_back({"h_start", p.off_hstart, B * K * D * N * 4});
            }
        } else if (bwd) {
            fail("backward not chunked", d, bwd);
        }
        check_regions(rs, u128(p.ws_total), d, bwd);
        if (p.mixed && (p.d4 <= 0 || p.d4 >= p.D || p.d4 % 64 != 0 || p.nb4 * 64 != p.d4))
            fail("mixed split", d, bwd);
    }
}

void check_block(const ss_block_dims& bd) {
    ss::BlockPlan bp;
    ++g_cases;
    if (ss::make_block_plan(bd, &bp) != SS_OK) return;
    const u128 M = u128(bp.M), D = u128(bp.D), N = u128(bp.N);
    std::vector<Region> rs{{"x", bp.off_x, M * D * 4},     {"z", bp.off_z, M * D * 4},
                           {"dt", bp.off_dt, M * 4},       {"B", bp.off_B, M * N * 4},
                           {"C", bp.off_C, M * N * 4},     {"partials", bp.off_part, u128(bp.S) * M * (1 + 2 * N) * 4},
                           {"scan", bp.off_scan, u128(bp.scan_ws)}};
    check_regions(rs, u128(bp.total), bp.sd, 0);
    if (bp.S < 1 || ss::xproj_split_len(bp.D, bp.S) * bp.S < bp.D) fail("splits", bp.sd, 0);
}

ss_dims dims(int64_t B, int64_t L, int64_t D, int64_t N, int dt = SS_BF16, int plan = 0,
             int64_t chunk = 0, int layout = 0, int disc = 0, int order = 0, int dtl = 0) {
    return ss_dims{B, L, D, N, dt, plan, chunk, layout, disc, order, dtl};
}

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t rnd(uint64_t n) {   // xorshift64*, uniform enough for picking cases
    g_rng ^= g_rng >> 12; g_rng ^= g_rng << 25; g_rng ^= g_rng >> 27;
    return (g_rng * 0x2545F4914F6CDD1Dull) % n;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc > 1) {
        // self-test of the checks: a region reaching past the workspace and two overlapping
        // regions must both be reported (the caller expects exit status 1 and "FAIL")
        const ss_dims d = dims(1, 64, 64, 16);
        check_regions({{"inside", 0, 256}, {"planted overlap", 0, 512}}, 1024, d, 0);
        return 0;
    }
    // the benchmark workloads and the decode-step shape
    const int64_t shapes[][4] = {{1, 256, 64, 16},      {2, 2048, 1536, 16}, {8, 2048, 5120, 16},
                                 {1, 1048576, 256, 16}, {4, 4096, 2048, 16}, {256, 1, 5120, 16}};
    for (const auto& s : shapes)
        for (int order = 0; order < 2; ++order)
            for (int dtl = 0; dtl < 2; ++dtl)
                for (int disc = 0; disc < 2; ++disc)
                    check_scan(dims(s[0], s[1], s[2], s[3], SS_BF16, 0, 0, 0, disc, order, dtl));
    // past 2^31 elements (buffers past 4 GB): the large-size GPU shapes and bigger ones
    const int64_t big[][4] = {{2, 1048600, 1100, 16}, {1, 2000000, 1100, 16}, {1, 1100000, 2100, 16},
                              {64, 1 << 20, 4096, 16}, {1, 1 << 26, 256, 64}, {16, 65536, 8192, 32}};
    for (const auto& s : big)
        for (int order = 0; order < 2; ++order)
            for (int plan = 0; plan < 3; ++plan)
                for (int layout = 0; layout < 4; ++layout)
                    check_scan(dims(s[0], s[1], s[2], s[3], SS_BF16, plan, 0, layout, 0, order, 0));
    // the block workload and a larger one
    check_block(ss_block_dims{8, 2048, 2560, 5120, 16, 0, 0});
    check_block(ss_block_dims{16, 8192, 4096, 8192, 64, 0, 0});
    // seeded sweep of the option space
    const int64_t Ns[] = {1, 2, 4, 8, 16, 32, 64};
    for (int i = 0; i < 20000; ++i) {
        const int64_t B = 1 + rnd(300), L = 1 + rnd(i % 4 == 0 ? 5000000 : 3000);
        const int64_t D = 1 + rnd(i % 5 == 0 ? 70000 : 3000), N = Ns[rnd(7)];
        const int64_t chunk = rnd(3) == 0 ? 8 * int64_t(rnd(20)) : 0;
        check_scan(dims(B, L, D, N, int(rnd(2)), int(rnd(3)), chunk, int(rnd(4)), int(rnd(2)),
                        int(rnd(2)), int(rnd(2))));
        if (i % 50 == 0)
            check_block(ss_block_dims{B, L, 8 * (1 + int64_t(rnd(1000))), 4 * (1 + int64_t(rnd(2000))), N,
                                      int(rnd(3)), int(rnd(4))});
    }
    // invalid and overflowing dims: errors, no arithmetic past the limits
    const int64_t bad[][4] = {{0, 1, 1, 16},          {1, 0, 1, 16},         {1, 1, -5, 16},
                              {1, 1, 1, 3},           {1, 1, 1, 128},        {INT64_MAX, 2, 2, 16},
                              {2, INT64_MAX, 2, 16},  {1 << 20, 1 << 20, 1 << 20, 16},
                              {INT64_MAX, INT64_MAX, INT64_MAX, 64}, {70000, 1, 1, 16}};
    for (const auto& s : bad)
        for (int bwd = 0; bwd < 2; ++bwd) {
            ss::Plan p;
            ++g_cases;
            if (ss::make_plan(dims(s[0], s[1], s[2], s[3]), bwd ? ss::kPlanBwd : ss::kPlanFwd, &p) == SS_OK)
                fail("invalid dims accepted", dims(s[0], s[1], s[2], s[3]), bwd);
        }
    ss::BlockPlan bp;
    ++g_cases;
    if (ss::make_block_plan(ss_block_dims{INT64_MAX, INT64_MAX, 8, 4, 16, 0, 0}, &bp) == SS_OK)
        fail("block overflow accepted", dims(0, 0, 0, 0), 0);
    std::printf("plan bounds ok %d\n", g_cases);
    return 0;
}
