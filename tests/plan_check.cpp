// Host-side check of the forward-pass plan (la_abi.cpp's make_fwd_plan) over
// random shapes: chunk and sub-chunk lengths are multiples of the block size,
// the chunk a multiple of the sub-chunk, sub-chunks at most 16384 tokens
// (unless one chunk covers the sequence), chunk rows within 2^30 bytes, and the
// slot counts match the dense shape; for packed input, over random and
// adversarial splits of the tokens into sequences, the chunk, sub-chunk and
// scan-tile counts the device derives from the lengths stay within the plan's
// bounds; explicit chunk / sub-chunk overrides are honoured when valid and
// rejected otherwise.  Built with g++ against stubs of the launchers; run by
// tests/test_plan_host.py.
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <random>
#include <vector>
#include "la_internal.h"
namespace la {
int launch_fwd(const FwdArgs &, void *, void *const *) { return 0; }
int launch_state_empty(const float *, float *, int, int, int, void *) { return 0; }
int read_cu_error(const FwdArgs &, void *, int *flag) { *flag = 0; return 0; }
int launch_decode(const void *, const void *, const void *, float *, void *, int, int, int, int, void *,
                  const int32_t *, int, int, double, const int32_t *) { return 0; }
int device_cu_count() { return 256; }
}
int main() {  // exit status 0 when every plan passes
    std::mt19937_64 rng(1);
    long bad = 0, n = 0;
    for (int it = 0; it < 200000; ++it) {
        int batch = 1 + rng() % 300, heads = 1 + rng() % 128;
        int d = (rng() & 1) ? 64 : 128, B = 64 << (rng() % 3);
        bool varlen = rng() & 1;
        int64_t L = 1 + (int64_t)(rng() % (1ull << (1 + rng() % 27)));
        if (varlen) L = L * (1 + rng() % 4);
        if (L > 2000000000LL) L = 2000000000LL;
        // whole GPUs and partitions of one (fewer compute units)
        const int cus = (rng() & 3) ? 256 : 32 + (int)(rng() % 225);
        la::FwdPlan p;
        if (la::make_fwd_plan(batch, heads, L, d, B, varlen, cus, la::PlanOverride{}, &p) != 0) {
            if (bad++ < 10) printf("planner rejected b=%d h=%d L=%lld\n", batch, heads, (long long)L);
            continue;
        }
        ++n;
        const int64_t cap = ((1LL << 30) / (d * 2)) / B * B;
        bool ok = p.chunk >= B && p.chunk % B == 0 && p.chunk <= cap && p.sub >= B && p.sub % B == 0 &&
                  p.chunk % p.sub == 0 && (p.sub <= 16384 || p.single_chunk) && p.bytes > 0;
        if (!varlen) {
            const int64_t cps = (L + p.chunk - 1) / p.chunk;
            ok = ok && p.nchunk_ub == batch * cps && p.single_chunk == (cps == 1);
        } else {
            // split L tokens into batch sequences: random cuts, or as many
            // sequences of C + 1 tokens as fit (the most sequences of two
            // chunks), or of 1 token (the most sequences)
            std::vector<int64_t> len(batch, 0);
            const int mode = rng() % 3;
            if (mode == 0) {
                std::vector<int64_t> cut(batch - 1);
                for (auto &x : cut) x = (int64_t)(rng() % (uint64_t)(L + 1));
                std::sort(cut.begin(), cut.end());
                int64_t prev = 0;
                for (int s = 0; s < batch - 1; ++s) { len[s] = cut[s] - prev; prev = cut[s]; }
                len[batch - 1] = L - prev;
            } else {
                const int64_t each = mode == 1 ? p.chunk + 1 : 1;
                int64_t left = L;
                for (int s = 0; s < batch - 1 && left >= each; ++s) { len[s] = each; left -= each; }
                len[batch - 1] += left;
            }
            int64_t sc = 0, su = 0, sg = 0, maxc = 0, maxs = 0;
            const int64_t R = p.chunk / p.sub;
            for (int64_t x : len) {   // the device's counts per sequence
                const int64_t nc = (x + p.chunk - 1) / p.chunk;
                const int64_t ns = nc >= 2 ? (nc - 1) * R + 1 : 0;
                sc += nc; su += ns; sg += (ns + p.scan_group - 1) / p.scan_group;
                maxc = std::max(maxc, nc);
                maxs = std::max(maxs, ns);
            }
            ok = ok && sc <= p.nchunk_ub && su <= p.nsub_ub && sg <= p.ntile_ub &&
                 (!p.single_chunk || maxc <= 1) &&
                 (p.scan_tiles || maxs <= p.scan_group);   // untiled: one tile per sequence
        }
        if (!ok && bad++ < 10)
            printf("bad: b=%d h=%d L=%lld d=%d B=%d varlen=%d -> C=%lld S=%lld single=%d\n", batch, heads,
                   (long long)L, d, B, (int)varlen, (long long)p.chunk, (long long)p.sub, (int)p.single_chunk);
    }
    // test-only overrides: a valid chunk / sub-chunk pair is taken as given,
    // anything else is rejected with LA_EINVAL (1) and leaves the plan alone
    for (int it = 0; it < 100000; ++it) {
        int batch = 1 + rng() % 50, heads = 1 + rng() % 64;
        int d = (rng() & 1) ? 64 : 128, B = 64 << (rng() % 3);
        bool varlen = rng() & 1;
        int64_t L = 1 + (int64_t)(rng() % (1ull << (1 + rng() % 22)));
        const int64_t cap = ((1LL << 30) / (d * 2)) / B * B;
        la::PlanOverride ov;
        ov.chunk = (rng() & 7) ? (int64_t)B * (1 + rng() % 300) : (int64_t)(1 + rng() % 70000);
        if (rng() & 1) ov.chunk = 16384 * (1 + rng() % 8);
        ov.sub = (rng() & 1) ? 0 : ((rng() & 3) ? ov.chunk / (1 + rng() % 4) : (int64_t)(1 + rng() % 5000));
        const bool cvalid = ov.chunk % B == 0 && ov.chunk <= cap && (ov.chunk <= 16384 || ov.chunk % 16384 == 0);
        const bool one = !varlen && (L + ov.chunk - 1) / ov.chunk == 1;
        const bool svalid = ov.sub == 0 || one || (ov.sub % B == 0 && ov.chunk % ov.sub == 0);
        la::FwdPlan p;
        p.chunk = -7;
        const int st = la::make_fwd_plan(batch, heads, L, d, B, varlen, 256, ov, &p);
        ++n;
        bool ok;
        if (cvalid && svalid) {
            ok = st == 0 && p.chunk == ov.chunk &&
                 p.sub == (one ? ov.chunk : (ov.sub ? ov.sub : std::min<int64_t>(ov.chunk, 16384)));
        } else {
            ok = st == 1 && p.chunk == -7;
        }
        if (!ok && bad++ < 10)
            printf("override: b=%d L=%lld B=%d C=%lld S=%lld varlen=%d -> st=%d C=%lld S=%lld\n", batch,
                   (long long)L, B, (long long)ov.chunk, (long long)ov.sub, (int)varlen, st,
                   (long long)p.chunk, (long long)p.sub);
    }
    printf("%ld plans, %ld bad\n", n, bad);
    return bad != 0;
}
